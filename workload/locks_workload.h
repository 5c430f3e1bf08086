/*
 * Seeded synthetic decode-step workloads for page-local key summaries.
 *
 * This module only makes inputs: queries, a paged K/V pool with locally
 * low-rank keys, planted "carrier" tokens and a shuffled block table.  It
 * holds none of the method's arithmetic (no summaries, no log-sum-exp, no
 * selection, no attention).  The oracle and the GPU library read the same
 * buffers it writes.
 *
 * Randomness is counter based: every value is a pure function of
 * (seed, tag, coordinates), built from the SplitMix64 finaliser (Steele,
 * Lea and Flood, "Fast splittable pseudorandom number generators", 2014)
 * and the Box-Muller transform, so results do not depend on thread count
 * or on the C library.
 *
 * Key model (the pages' observation that attention keys are locally
 * low-rank though globally high-rank; "LOCKS", abstract, and the gist.science
 * technical summary, section 3 "Localiteit van Structuur"):
 *   for every (sequence b, KV head g, logical page j) an independent
 *   orthonormal basis Q (d x m) is drawn; token i of the page gets
 *   k_i = Q z_i + e_i (+ o_page), z_{i,t} ~ N(0, (2^-t)^2), e ~ N(0, noise^2).
 * Carriers: per (b, g), n_c distinct full pages each get one token replaced
 * by a key aligned with the group's mean query direction (cosine 0.9 at
 * gain 1), the "carrier pages" the pages say selection must keep.
 */
#ifndef LOCKS_WORKLOAD_H
#define LOCKS_WORKLOAD_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct {
    int32_t batch;          /* B */
    int32_t num_q_heads;    /* H_q */
    int32_t num_kv_heads;   /* H_kv, divides H_q */
    int32_t head_dim;       /* d */
    int32_t page_size;      /* P tokens per page */
    int32_t subspace_rank;  /* m, rank of each page's key subspace (<= d) */
    int32_t carriers;       /* n_c carrier pages per (b, g) */
    int32_t kv_bf16;        /* 1: K/V written as bf16 bit patterns (uint16); 0: float32 */
    int32_t poison_tail;    /* 1: unused slots of a partial last page hold NaN */
    int32_t num_threads;    /* <= 0: OpenMP default */
    double noise_std;       /* std of the i.i.d. key noise */
    double page_offset_std; /* std of a per-page key offset (0 = none) */
    double carrier_gain;    /* gamma: carrier norm = gamma * norm of the replaced key */
    double carrier_cos;     /* cosine between a carrier key and the group query direction */
    double q_std;           /* std of query elements */
    double v_std;           /* std of value elements */
    uint64_t seed;
} wl_params;

/* Number of pages sequence b occupies: ceil(seq_len / P). */
int32_t wl_pages_for(int32_t seq_len, int32_t page_size);

/*
 * Fill every buffer.  Sizes, with NB = sum_b ceil(seq_lens[b] / P) and
 * max_pages >= max_b ceil(seq_lens[b] / P):
 *   q             [B][H_q][d]            float32
 *   k, v          [NB][H_kv][P][d]       float32 or bf16 bits (kv_bf16)
 *   block_table   [B][max_pages]         int32; logical page -> physical block, -1 past the end
 *   carrier_page  [B][H_kv][n_c]         int32 logical page of each carrier (sorted ascending)
 *   carrier_slot  [B][H_kv][n_c]         int32 token slot of each carrier in its page
 * carrier_page/carrier_slot may be NULL when n_c == 0.
 * Returns 0 on success, a negative code on invalid parameters
 * (-1 shapes, -2 not enough full pages for the carriers, -3 allocation).
 */
int wl_generate(const wl_params* p, const int32_t* seq_lens, int32_t max_pages,
                int32_t num_blocks, float* q, void* k, void* v, int32_t* block_table,
                int32_t* carrier_page, int32_t* carrier_slot);

/* Building blocks, exported for the generator's own tests. */
uint64_t wl_splitmix64(uint64_t x);
uint64_t wl_hash(uint64_t seed, uint64_t tag, uint64_t a, uint64_t b, uint64_t c, uint64_t e);
double wl_normal(uint64_t h);            /* standard normal from one 64-bit hash */
double wl_uniform(uint64_t h);           /* uniform in [0, 1) from one 64-bit hash */
uint16_t wl_f32_to_bf16(float x);        /* round to nearest even */
float wl_bf16_to_f32(uint16_t b);

#ifdef __cplusplus
}
#endif
#endif
