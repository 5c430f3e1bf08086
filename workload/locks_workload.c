/*
 * Seeded synthetic decode-step workloads; see locks_workload.h.
 * Input generation only: nothing here computes a summary, a log-sum-exp,
 * a selection or an attention output.
 */
#include "locks_workload.h"

#include <math.h>
#include <omp.h>
#include <stdlib.h>
#include <string.h>

enum {
    TAG_Q = 1,
    TAG_BASIS = 2,
    TAG_Z = 3,
    TAG_NOISE = 4,
    TAG_OFFSET = 5,
    TAG_V = 6,
    TAG_PERM = 7,
    TAG_CARRIER_PICK = 8,
    TAG_CARRIER_SLOT = 9,
    TAG_CARRIER_DIR = 10,
};

uint64_t wl_splitmix64(uint64_t x) {
    uint64_t z = x + 0x9e3779b97f4a7c15ULL;
    z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ULL;
    z = (z ^ (z >> 27)) * 0x94d049bb133111ebULL;
    return z ^ (z >> 31);
}

uint64_t wl_hash(uint64_t seed, uint64_t tag, uint64_t a, uint64_t b, uint64_t c, uint64_t e) {
    uint64_t x = wl_splitmix64(seed);
    x = wl_splitmix64(x ^ tag);
    x = wl_splitmix64(x ^ a);
    x = wl_splitmix64(x ^ b);
    x = wl_splitmix64(x ^ c);
    return wl_splitmix64(x ^ e);
}

double wl_uniform(uint64_t h) { return (double)(h >> 11) * 0x1.0p-53; }

double wl_normal(uint64_t h) {
    /* Box-Muller, cosine branch; u1 in (0, 1) so the log is finite. */
    const double u1 = ((double)(h >> 11) + 0.5) * 0x1.0p-53;
    const double u2 = wl_uniform(wl_splitmix64(h));
    return sqrt(-2.0 * log(u1)) * cos(6.283185307179586476925 * u2);
}

uint16_t wl_f32_to_bf16(float x) {
    uint32_t u;
    memcpy(&u, &x, 4);
    if ((u & 0x7f800000u) == 0x7f800000u && (u & 0x007fffffu)) return (uint16_t)((u >> 16) | 0x40);
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

float wl_bf16_to_f32(uint16_t b) {
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, 4);
    return f;
}

int32_t wl_pages_for(int32_t seq_len, int32_t page_size) {
    return (seq_len + page_size - 1) / page_size;
}

/* Store one element of K or V, rounding double -> float (-> bf16). */
static void store_elem(void* base, int bf16, size_t idx, double x) {
    const float f = (float)x;
    if (bf16)
        ((uint16_t*)base)[idx] = wl_f32_to_bf16(f);
    else
        ((float*)base)[idx] = f;
}

/* Orthonormal d x m basis (column t at basis[t*d ..]) by two passes of
 * modified Gram-Schmidt over Gaussian columns. */
static void page_basis(const wl_params* p, int b, int g, int j, double* basis) {
    const int d = p->head_dim, m = p->subspace_rank;
    for (int t = 0; t < m; ++t) {
        double* col = basis + (size_t)t * d;
        for (int e = 0; e < d; ++e)
            col[e] = wl_normal(wl_hash(p->seed, TAG_BASIS, b, g, j, (uint64_t)t * d + e));
        for (int pass = 0; pass < 2; ++pass) {
            for (int s = 0; s < t; ++s) {
                const double* prev = basis + (size_t)s * d;
                double dot = 0.0;
                for (int e = 0; e < d; ++e) dot += prev[e] * col[e];
                for (int e = 0; e < d; ++e) col[e] -= dot * prev[e];
            }
        }
        double nrm = 0.0;
        for (int e = 0; e < d; ++e) nrm += col[e] * col[e];
        nrm = sqrt(nrm);
        for (int e = 0; e < d; ++e) col[e] /= nrm;
    }
}

/* Token i of logical page j of (b, g), before any carrier replacement. */
static void page_key(const wl_params* p, int b, int g, int j, int i, const double* basis,
                     double* key) {
    const int d = p->head_dim, m = p->subspace_rank;
    for (int e = 0; e < d; ++e) key[e] = 0.0;
    double scale = 1.0;
    for (int t = 0; t < m; ++t, scale *= 0.5) {
        const double z =
            scale * wl_normal(wl_hash(p->seed, TAG_Z, b, g, j, (uint64_t)i * m + t));
        const double* col = basis + (size_t)t * d;
        for (int e = 0; e < d; ++e) key[e] += z * col[e];
    }
    for (int e = 0; e < d; ++e) {
        key[e] += p->noise_std *
                  wl_normal(wl_hash(p->seed, TAG_NOISE, b, g, j, (uint64_t)i * d + e));
        if (p->page_offset_std != 0.0)
            key[e] += p->page_offset_std *
                      wl_normal(wl_hash(p->seed, TAG_OFFSET, b, g, j, (uint64_t)e));
    }
}

typedef struct {
    int32_t page;
    int32_t slot;
} carrier_t;

static int cmp_carrier(const void* a, const void* b) {
    const carrier_t* x = (const carrier_t*)a;
    const carrier_t* y = (const carrier_t*)b;
    return (x->page > y->page) - (x->page < y->page);
}

int wl_generate(const wl_params* p, const int32_t* seq_lens, int32_t max_pages,
                int32_t num_blocks, float* q, void* k, void* v, int32_t* block_table,
                int32_t* carrier_page, int32_t* carrier_slot) {
    const int B = p->batch, Hq = p->num_q_heads, Hkv = p->num_kv_heads;
    const int d = p->head_dim, P = p->page_size, m = p->subspace_rank, nc = p->carriers;
    if (B <= 0 || Hq <= 0 || Hkv <= 0 || Hq % Hkv || d <= 0 || P <= 0 || m < 0 || m > d ||
        nc < 0)
        return -1;
    const int G = Hq / Hkv;

    /* Page bookkeeping: first physical slot of each sequence in the permutation. */
    int64_t total = 0;
    int32_t* page_off = (int32_t*)malloc(sizeof(int32_t) * (size_t)(B + 1));
    if (!page_off) return -3;
    for (int b = 0; b < B; ++b) {
        if (seq_lens[b] < 0) { free(page_off); return -1; }
        const int32_t np = wl_pages_for(seq_lens[b], P);
        if (np > max_pages) { free(page_off); return -1; }
        if (nc > seq_lens[b] / P) { free(page_off); return -2; }
        page_off[b] = (int32_t)total;
        total += np;
    }
    page_off[B] = (int32_t)total;
    if (total != num_blocks) { free(page_off); return -1; }

    /* Block table: a seeded random permutation of the physical blocks. */
    int32_t* perm = (int32_t*)malloc(sizeof(int32_t) * (size_t)(total > 0 ? total : 1));
    if (!perm) { free(page_off); return -3; }
    for (int64_t i = 0; i < total; ++i) perm[i] = (int32_t)i;
    for (int64_t i = total - 1; i > 0; --i) {
        const int64_t r =
            (int64_t)(wl_uniform(wl_hash(p->seed, TAG_PERM, 0, 0, 0, (uint64_t)i)) * (double)(i + 1));
        const int32_t t = perm[i];
        perm[i] = perm[r];
        perm[r] = t;
    }
    for (int b = 0; b < B; ++b) {
        const int32_t np = page_off[b + 1] - page_off[b];
        for (int j = 0; j < max_pages; ++j)
            block_table[(size_t)b * max_pages + j] = j < np ? perm[page_off[b] + j] : -1;
    }

    /* Queries. */
    for (int b = 0; b < B; ++b)
        for (int h = 0; h < Hq; ++h)
            for (int e = 0; e < d; ++e)
                q[((size_t)b * Hq + h) * d + e] =
                    (float)(p->q_std * wl_normal(wl_hash(p->seed, TAG_Q, b, h, 0, e)));

    /* Carrier placement per (b, g): a partial Fisher-Yates over the full pages. */
    carrier_t* carriers = NULL;
    if (nc > 0) {
        carriers = (carrier_t*)malloc(sizeof(carrier_t) * (size_t)B * Hkv * nc);
        if (!carriers) { free(perm); free(page_off); return -3; }
        for (int b = 0; b < B; ++b) {
            const int32_t full = seq_lens[b] / P;
            int32_t* idx = (int32_t*)malloc(sizeof(int32_t) * (size_t)full);
            if (!idx) { free(carriers); free(perm); free(page_off); return -3; }
            for (int g = 0; g < Hkv; ++g) {
                for (int32_t i = 0; i < full; ++i) idx[i] = i;
                carrier_t* out = carriers + ((size_t)b * Hkv + g) * nc;
                for (int c = 0; c < nc; ++c) {
                    const double u = wl_uniform(wl_hash(p->seed, TAG_CARRIER_PICK, b, g, 0, c));
                    const int32_t r = c + (int32_t)(u * (double)(full - c));
                    const int32_t t = idx[c];
                    idx[c] = idx[r];
                    idx[r] = t;
                    out[c].page = idx[c];
                    out[c].slot = (int32_t)(
                        wl_uniform(wl_hash(p->seed, TAG_CARRIER_SLOT, b, g, c, 0)) * (double)P);
                }
                qsort(out, (size_t)nc, sizeof(carrier_t), cmp_carrier);
                for (int c = 0; c < nc; ++c) {
                    if (carrier_page) carrier_page[((size_t)b * Hkv + g) * nc + c] = out[c].page;
                    if (carrier_slot) carrier_slot[((size_t)b * Hkv + g) * nc + c] = out[c].slot;
                }
            }
            free(idx);
        }
    }

    /* Keys and values, one (b, page, g) unit per iteration. */
    const int64_t units = total * Hkv;
    int status = 0;
#pragma omp parallel num_threads(p->num_threads > 0 ? p->num_threads : omp_get_max_threads())
    {
        double* basis = (double*)malloc(sizeof(double) * (size_t)d * (m > 0 ? m : 1));
        double* key = (double*)malloc(sizeof(double) * (size_t)d);
        double* dir = (double*)malloc(sizeof(double) * (size_t)d);
        if (!basis || !key || !dir) {
#pragma omp atomic write
            status = -3;
        }
#pragma omp for schedule(dynamic, 16)
        for (int64_t u = 0; u < units; ++u) {
            if (!basis || !key || !dir) continue;
            const int g = (int)(u % Hkv);
            const int64_t gp = u / Hkv; /* global page in sequence order */
            int b = 0;
            while (gp >= page_off[b + 1]) ++b;
            const int j = (int)(gp - page_off[b]);
            const int32_t phys = block_table[(size_t)b * max_pages + j];
            const int32_t valid =
                seq_lens[b] - j * P < P ? seq_lens[b] - j * P : P; /* tokens in this page */
            const size_t base = ((size_t)phys * Hkv + g) * (size_t)P * d;

            if (m > 0) page_basis(p, b, g, j, basis);
            const carrier_t* pc = carriers ? carriers + ((size_t)b * Hkv + g) * nc : NULL;
            for (int i = 0; i < P; ++i) {
                const size_t row = base + (size_t)i * d;
                if (i >= valid) {
                    const double fill = p->poison_tail ? NAN : 0.0;
                    for (int e = 0; e < d; ++e) {
                        store_elem(k, p->kv_bf16, row + e, fill);
                        store_elem(v, p->kv_bf16, row + e, fill);
                    }
                    continue;
                }
                page_key(p, b, g, j, i, basis, key);
                for (int c = 0; pc && c < nc; ++c) {
                    if (pc[c].page != j || pc[c].slot != i) continue;
                    /* Carrier: gain * |k| * (cos * qhat + sin * w), w a unit vector
                     * orthogonal to the group's mean query direction qhat. */
                    double qn = 0.0;
                    for (int e = 0; e < d; ++e) {
                        double s = 0.0;
                        for (int h = g * G; h < (g + 1) * G; ++h)
                            s += (double)q[((size_t)b * Hq + h) * d + e];
                        dir[e] = s;
                        qn += s * s;
                    }
                    qn = sqrt(qn);
                    for (int e = 0; e < d; ++e) dir[e] /= qn;
                    double knorm = 0.0;
                    for (int e = 0; e < d; ++e) knorm += key[e] * key[e];
                    knorm = sqrt(knorm);
                    /* random direction, made orthogonal to qhat (kept in key[] temporarily) */
                    double proj = 0.0;
                    for (int e = 0; e < d; ++e) {
                        key[e] = wl_normal(wl_hash(p->seed, TAG_CARRIER_DIR, b, g, c, e));
                        proj += key[e] * dir[e];
                    }
                    double wn = 0.0;
                    for (int e = 0; e < d; ++e) {
                        key[e] -= proj * dir[e];
                        wn += key[e] * key[e];
                    }
                    wn = sqrt(wn);
                    const double cs = p->carrier_cos, sn = sqrt(1.0 - cs * cs);
                    for (int e = 0; e < d; ++e)
                        key[e] = knorm * p->carrier_gain * (cs * dir[e] + sn * key[e] / wn);
                }
                for (int e = 0; e < d; ++e) {
                    store_elem(k, p->kv_bf16, row + e, key[e]);
                    store_elem(v, p->kv_bf16, row + e,
                               p->v_std * wl_normal(wl_hash(p->seed, TAG_V, b, g, j,
                                                            (uint64_t)i * d + e)));
                }
            }
        }
        free(basis);
        free(key);
        free(dir);
    }
    free(carriers);
    free(perm);
    free(page_off);
    return status;
}
