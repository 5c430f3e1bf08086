// Kernel templates of the summary scan, instantiated once per stored
// summary type by scan_f32.hip, scan_bf16.hip and scan_q8q4.hip (one
// translation unit each, so they compile in parallel); scan.hip dispatches.
//
// Summary scan: per-page estimated attention mass from the resident summary
// alone (gist.science technical summary, section 2, Reconstructie en
// Selectie, displayed estimator), aggregated over each GQA group by
// log-sum-exp (section 2, Group-Shared Selection, read as the sum of the
// heads' unnormalised masses).
//
// For page j of (b, g) and head h of the group, in log2 units with q
// pre-scaled by log2(e)/sqrt(d):
//   T[k][h]   = basis_k . q_h                       (MFMA 16x16x4 fp32)
//   beta[h]   = mu . q_h                            (MFMA, 16 pages per tile)
//   L[i][h]   = sum_k coef[i][k] T[k][h]            (MFMA 16x16x4 fp32)
//   s2[h]     = beta[h] + log2 sum_i 2^L[i][h]      (VALU: max, exp2, sum)
//   a2        = log2 sum_h 2^s2[h]                  (VALU, 16-lane row)
// and the outputs are s2 * ln 2 and a2 * ln 2.  bf16 and integer-code
// summaries run the same products on the bf16 matrix cores (below).
//
// One wave scans 16 consecutive logical pages of one (b, g).  Its query
// fragment (16 heads x d; heads >= G load head 0 and scale it by 0) stays in
// registers.  All loads
// are 16-byte vector loads; each MFMA operand is taken straight from the
// loaded registers thanks to the free choice of contraction order:
// MFMA step s of a tile contracts d = 16*(s/4) + 4*(l/16) + s%4, so lane l
// loads d-chunks [16t + 4*(l/16), +4) of its row (64 contiguous bytes per
// row per load instruction).
// When asked, the wave also writes the largest page mass of its 16 pages
// (the run maximum the top-k uses to skip runs that cannot hold a winner).
#pragma once

#include <type_traits>

#include "device_common.hpp"
#include "launchers.hpp"

namespace locks {

namespace {

// A wave scans NP consecutive pages (NP a multiple of kRunPages: whole runs)
// with PF basis tiles in flight ahead of the one computed; the launcher picks
// them per workload.  The bf16 and integer-code paths use one run, one tile.
constexpr int kBatch = kRunPages;  // pages per wave of the bf16 / code paths
constexpr int kPrefetch = 1;       // the bf16 path's tiles in flight ahead
constexpr int kCodePrefetch = 2;   // the code path's (its tiles are small: more in flight)
constexpr int kChains = 2;         // independent accumulator chains of an fp32 d contraction

// State of one wave's batch, shared by the two specialisations below.
template <int D>
struct WaveCtx {
    int b, g, j0, G, Hkv, r, lane, w, c;
    bool head_ok;
    int my_phys;  // lane l: block of page j0 + l % NP (-1: absent)
    float* out_page;
    float qf[D / 4];  // query words as loaded (head c, or head 0 for padding heads)
    float qs;         // scale to log2 units, 0 for padding heads
};

// Summary element types: fp32, bf16 bit patterns (uint16_t), or int8 / int4
// codes (int8_t).  E = elements per lane and 32-wide d chunk of the query
// fragment (16-byte loads for fp32 and bf16; the codes reuse bf16's layout).
template <typename TS>
struct Summ {
    static constexpr int E = 16 / (int)sizeof(TS);
};
template <>
struct Summ<int8_t> {
    static constexpr int E = 8;
};

// Address of element `off` of `base`.  kOff32: every summary array is below
// 4 GiB, so the byte offset is a 32-bit value added to the uniform base (one
// VALU op per address instead of 64-bit arithmetic).
template <typename TS, bool kOff32>
__device__ __forceinline__ const char* elem_addr(const void* base, size_t off) {
    if constexpr (kOff32)
        return static_cast<const char*>(base) + (uint32_t)((uint32_t)off * (uint32_t)sizeof(TS));
    else
        return static_cast<const char*>(base) + off * sizeof(TS);
}

// N (1, 2 or 4) consecutive fp32 summary elements starting at element `off`.
template <bool kOff32, int N>
__device__ __forceinline__ void load_f32(const void* base, size_t off, float* out) {
    const char* ptr = elem_addr<float, kOff32>(base, off);
    if constexpr (N == 1) {
        out[0] = *reinterpret_cast<const float*>(ptr);
    } else if constexpr (N == 2) {
        const f32x2 v = *reinterpret_cast<const f32x2*>(ptr);
        out[0] = v[0];
        out[1] = v[1];
    } else {
        static_assert(N == 4, "loads of 1, 2 or 4 elements");
        const f32x4 v = *reinterpret_cast<const f32x4*>(ptr);
#pragma unroll
        for (int e = 0; e < 4; ++e) out[e] = v[e];
    }
}

// Per-page tail of batches whose logits arrive shifted: the coefficient
// product starts from beta - shift, shift = the page's largest beta over the
// group's heads (a wave-uniform value).  Lane (w, c) holds the shifted logits
// of tokens 16 mt + 4w + v for head c (log2 units) in L[mt][v], every lane
// the same page; padding heads carry values near -1e30 and drop out.
// Log-sum-exp over the group is the log-sum-exp of all 64 x 16 (token, head)
// logits of the page.  The coefficients of a page sum to zero over its tokens
// (they are projections of keys less their mean), so the best head's largest
// shifted logit is about 0 or more and the sum of 2^logit is at least about 1;
// it exceeds 2^60 only for deviations from the centroid term of some 50 log2
// units.  Pages whose sum leaves [2^-60, 2^60] take the exact form (the
// page's max subtracted first).  With per-head output (kHeads) every head's
// sum is taken with its own max.
template <int MT, bool kHeads, bool kMasked, int D>
__device__ __forceinline__ void page_mass_shifted(const ScanParams& a, const WaveCtx<D>& x,
                                                  const f32x4* L, int pb, float shift,
                                                  float& run_mx) {
    const int j = x.j0 + pb;
    auto local_max = [&]() {
        float m = L[0][0];
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int v = 0; v < 4; ++v) m = fmaxf(m, L[mt][v]);
        return m;
    };
    auto local_sum = [&](float off) {
        float s = fast_exp2(L[0][0] - off);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int v = (mt == 0 ? 1 : 0); v < 4; ++v) s += fast_exp2(L[mt][v] - off);
        return s;
    };
    float a2, s2 = 0.0f;
    if constexpr (!kHeads) {
        const float sum = sum_in_row(sum_over_rows(local_sum(0.0f)));
        if (sum >= 0x1p-60f && sum <= 0x1p60f) {
            a2 = shift + fast_log2(sum);
        } else {
            const float mx = max_in_row(max_over_rows(local_max()));
            a2 = shift + mx + fast_log2(sum_in_row(sum_over_rows(local_sum(mx))));
        }
    } else {
        const float mx = max_over_rows(local_max());
        s2 = shift + mx + fast_log2(sum_over_rows(local_sum(mx)));
        const float xv = x.head_ok ? s2 : -INFINITY;
        const float gm = max_in_row(xv);
        a2 = gm + fast_log2(sum_in_row(x.head_ok ? fast_exp2(xv - gm) : 0.0f));
    }
    if (j < a.max_pages) {
        const bool ok = !kMasked || __builtin_amdgcn_readlane(x.my_phys, pb) >= 0;
        const float mass = ok ? a2 * kLn2 : -INFINITY;
        run_mx = fmaxf(run_mx, mass);
        if (x.lane == 0) x.out_page[j] = mass;
        if constexpr (kHeads) {
            if (x.w == 0 && x.head_ok)
                a.head_logmass[((size_t)x.b * a.num_q_heads + x.g * x.G + x.c) * a.max_pages + j] =
                    ok ? s2 * kLn2 : -INFINITY;
        }
    }
}

// Shifted centroid terms for page_mass_shifted, from the beta tiles of NR
// runs (lane (w, c) element v of beta[n]: page 16n + 4w + v, head c; padding
// heads are given -1e30): each lane receives beta - shift of all 16 NR pages
// for its head in betas[], through a per-wave LDS table tbl[16][16 NR], and
// lane (w, c) keeps the shifts of pages 16n + 4w + v in sv[n][v].
template <int NR>
__device__ __forceinline__ void shift_betas(const f32x4* beta, bool head_ok, int w, int c,
                                            float (*tbl)[16 * NR], float* betas, float (*sv)[4]) {
#pragma unroll
    for (int n = 0; n < NR; ++n) {
        f32x4 bt = beta[n];
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            bt[v] = head_ok ? bt[v] : -1e30f;
            sv[n][v] = max_in_row(bt[v]);
            bt[v] -= sv[n][v];
        }
        *reinterpret_cast<f32x4*>(&tbl[c][16 * n + 4 * w]) = bt;
    }
    // the wave's LDS writes are done before its reads of other lanes' entries
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
    for (int n4 = 0; n4 < 4 * NR; ++n4) {
        const f32x4 v = *reinterpret_cast<const f32x4*>(&tbl[c][4 * n4]);
#pragma unroll
        for (int e = 0; e < 4; ++e) betas[4 * n4 + e] = v[e];
    }
}
// The shift of page pb of the batch, wave-uniform (held by lane 16 ((pb%16)/4)).
__device__ __forceinline__ float page_shift(const float (*sv)[4], int pb) {
    return __int_as_float(
        __builtin_amdgcn_readlane(__float_as_int(sv[pb / 16][pb & 3]), 16 * ((pb & 15) >> 2)));
}

// The query words, passed through empty asm statements that clobber memory:
// they stay after every load issued before them, and the query's arithmetic
// stays after them, so a wave's first summary loads go out before it waits
// for its query.
template <int N>
__device__ __forceinline__ void query_after_loads(const float* qf, float* qv) {
#pragma unroll
    for (int i = 0; i < N; ++i) {
        qv[i] = qf[i];
        asm volatile("" : "+v"(qv[i])::"memory");
    }
}
// The same for loaded summary words that are used before the first tile.
template <typename T>
__device__ __forceinline__ void after_loads(T& v) {
    asm volatile("" : "+v"(v)::"memory");
}

// One wave's batch of NP pages (NP / 16 runs).  kMasked: some page of the
// batch is absent or the rank is padded, so loads are zeroed per row;
// otherwise no masking code is emitted.  kHeads: per-head masses are written
// too.  fp32 summaries: the word layout keeps the fp32 loads 64 contiguous
// bytes per row; the contraction order of the MFMA steps is chosen to match
// it.  PF basis tiles are in flight ahead of the one computed, across run
// boundaries.
template <int P, int D, int RR, bool kExact, bool kHeads, bool kOff32, bool kMasked, int NP,
          int PF>
__device__ __forceinline__ void scan_batch_f32(const ScanParams& a, const WaveCtx<D>& x) {
    using TS = float;
    constexpr int PPT = 16 / RR;          // pages per basis tile (16 rows = PPT pages x RR rows)
    constexpr int NTILE = NP / PPT;       // basis tiles per batch
    constexpr int NRUN = NP / kRunPages;  // runs per batch
    constexpr int KS2 = RR / 4;           // K-steps of the coefficient product
    constexpr int MT = P / 16;            // token tiles per page
    constexpr int DS = D / 4;             // words of a row held per lane
    constexpr int E = Summ<TS>::E;        // elements per 16-byte load
    constexpr int NCH = D / (4 * E);      // 16-byte loads per row and lane
    static_assert(NP % kRunPages == 0 && NP <= kWave && PF >= 1, "whole runs per wave");
    using Off = typename std::conditional<kOff32, uint32_t, size_t>::type;
    // the exact path's rank is the compile-time RR (address products become shifts)
    const int w = x.w, c = x.c, g = x.g, Hkv = x.Hkv, r = kExact ? RR : x.r;
    const int my_phys = x.my_phys;
    auto phys_at = [&](int pb) { return __shfl(my_phys, pb, kWave); };
    auto phys_uniform = [&](int pb) { return __builtin_amdgcn_readlane(my_phys, pb); };

    // The query in fp32, word s of lane (w, c) at d = 16 (s/4) + 4w + s%4
    // (the fp32 load layout): MFMA step s contracts these 4 d's.  Scaled once
    // the first tile's and the centroids' loads are issued (scaling waits for
    // the query's loads; the summary loads need not).
    float qv[DS];
    auto prepare_q = [&]() {
        query_after_loads<DS>(x.qf, qv);
#pragma unroll
        for (int i = 0; i < DS; ++i) qv[i] *= x.qs;
    };
    // (rows of A) . q for the lane's DS words: 16x16x4 fp32 steps in
    // kChains independent accumulator chains
    auto dot_q = [&](const uint32_t* words) {
        f32x4 acc[kChains];
#pragma unroll
        for (int i = 0; i < kChains; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int st = 0; st < DS; ++st)
            acc[st % kChains] = mfma_16x16x4_f32(__uint_as_float(words[st]), qv[st], acc[st % kChains]);
        f32x4 T = acc[0];
#pragma unroll
        for (int i = 1; i < kChains; ++i) T += acc[i];
        return T;
    };

    // Basis-tile row assignment for the loading lane (row m = c):
    //   page-in-tile p = (m%4) / KS2, k-step ks = (m%4) % KS2, basis row kk = KS2*(m/4) + ks.
    // After the MFMA, lane (w, c) element v holds T[page v/KS2][KS2*w + v%KS2][head c],
    // which is exactly its B operand for k-step v%KS2 of page v/KS2.
    const int a_pin = (c & 3) / KS2;
    const int a_kk = KS2 * (c >> 2) + ((c & 3) % KS2);

    // A tile keeps the loaded words as they are and reinterprets them where
    // the MFMAs consume them, so the waits for a tile's loads fall at its use.
    constexpr int CFW = KS2;  // words per coefficient chunk
    struct Tile {
        uint32_t v[DS];
        uint32_t cf[PPT][MT][CFW];
    };
    auto widen = [](const uint32_t* words, int i) -> float { return __uint_as_float(words[i]); };
    // Loads are unconditional (absent rows read a clamped, valid address and
    // are zeroed afterwards) so that the next tile's loads stay in flight
    // while the current tile is computed.
    auto load_tile = [&](int tt, Tile& T) {
        const int pj = phys_at(tt * PPT + a_pin);
        const bool row_ok = !kMasked || (pj >= 0 && a_kk < r);
        const Off src = (((Off)(kMasked && pj < 0 ? 0 : pj) * Hkv + g) * r +
                         (kMasked && a_kk >= r ? r - 1 : a_kk)) * D + E * w;
#pragma unroll
        for (int t = 0; t < NCH; ++t) {
            const u32x4 v = *reinterpret_cast<const u32x4*>(elem_addr<TS, kOff32>(a.basis, src + 4 * E * t));
#pragma unroll
            for (int e = 0; e < 4; ++e) T.v[4 * t + e] = row_ok ? v[e] : 0u;
        }
#pragma unroll
        for (int p = 0; p < PPT; ++p) {
            const int pp = phys_uniform(tt * PPT + p);
            const bool ok = !kMasked || pp >= 0;
            const Off csrc = ((Off)(kMasked && pp < 0 ? 0 : pp) * Hkv + g) * P * r;
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                const Off row = csrc + (Off)(16 * mt + c) * r;
                if (kExact || KS2 == 1) {
                    // KS2 consecutive elements k = KS2 w .. (rank not padded), or the
                    // single element k = w clamped to the rank and zeroed past it
                    const int k0 = kExact ? KS2 * w : (w < r ? w : r - 1);
                    const bool kok = kExact || w < r;
                    const char* ptr = elem_addr<TS, kOff32>(a.coef, row + k0);
                    if constexpr (CFW == 1) {
                        const uint32_t word = *reinterpret_cast<const uint32_t*>(ptr);
                        T.cf[p][mt][0] = (ok && kok) ? word : 0u;
                    } else if constexpr (CFW == 2) {
                        const u32x2 v = *reinterpret_cast<const u32x2*>(ptr);
                        T.cf[p][mt][0] = ok ? v[0] : 0u;
                        T.cf[p][mt][1] = ok ? v[1] : 0u;
                    } else {
                        const u32x4 v = *reinterpret_cast<const u32x4*>(ptr);
#pragma unroll
                        for (int e = 0; e < 4; ++e) T.cf[p][mt][e] = ok ? v[e] : 0u;
                    }
                } else {
                    // padded rank with KS2 > 1: element by element, clamped and
                    // zeroed past the rank
#pragma unroll
                    for (int e = 0; e < CFW; ++e) T.cf[p][mt][e] = 0u;
#pragma unroll
                    for (int ks = 0; ks < KS2; ++ks) {
                        const int kk = KS2 * w + ks;
                        const char* ptr = elem_addr<TS, kOff32>(a.coef, row + (kk < r ? kk : r - 1));
                        const uint32_t word = *reinterpret_cast<const uint32_t*>(ptr);
                        T.cf[p][mt][ks] = (ok && kk < r) ? word : 0u;
                    }
                }
            }
        }
    };
    // coefficient element ks of chunk (p, mt)
    auto coef_el = [&](const Tile& tl, int p, int mt, int ks) -> float {
        return widen(tl.cf[p][mt], ks);
    };

    // ring of tiles: the loads of tiles tt+1 .. tt+PF are in flight while
    // tile tt is computed
    Tile ring[PF + 1];
#pragma unroll
    for (int i = 0; i < PF && i < NTILE; ++i) load_tile(i, ring[i]);

    // beta tiles, one per run: A row m = page j0 + 16 n + m (lane column c
    // supplies row c).  All runs' centroid loads go out before the first product.
    f32x4 beta[NRUN];
    {
        uint32_t mv[NRUN][DS];
#pragma unroll
        for (int n = 0; n < NRUN; ++n) {
            const int pm = phys_at(16 * n + c);
            const Off src = ((Off)(pm < 0 ? 0 : pm) * Hkv + g) * D + E * w;
#pragma unroll
            for (int t = 0; t < NCH; ++t) {
                float v[E];
                load_f32<kOff32, E>(a.mu, src + 4 * E * t, v);
#pragma unroll
                for (int e = 0; e < E; ++e) mv[n][E * t + e] = __float_as_uint(v[e]);
            }
        }
        prepare_q();
#pragma unroll
        for (int n = 0; n < NRUN; ++n) {
            const int pm = phys_at(16 * n + c);
#pragma unroll
            for (int i = 0; i < DS; ++i) {
                after_loads(mv[n][i]);
                mv[n][i] = (!kMasked || pm >= 0) ? mv[n][i] : 0u;
            }
            beta[n] = dot_q(mv[n]);
        }
    }
    // lane (w, c) now holds beta[page j0 + 16 n + 4w + v][head c] in element v
    // of beta[n].  The coefficient products start from beta - shift, shift =
    // the page's largest beta over the group's heads (page_mass_shifted): the
    // shifts stay in sv[n][v] of lane (w, c), and a per-wave table in LDS hands
    // every lane beta - shift of all NP pages for its head.
    float sv[NRUN][4];
    float betas[NP];
    {
        __shared__ float tbl[4][16][NP];  // [wave of the block][head][page]
        shift_betas<NRUN>(beta, x.head_ok, w, c, tbl[threadIdx.x >> 6], betas, sv);
    }

    float run_mx = -INFINITY;  // max of the written page masses of the current run
#pragma unroll
    for (int tt = 0; tt < NTILE; ++tt) {
        if (tt + PF < NTILE) load_tile(tt + PF, ring[(tt + PF) % (PF + 1)]);
        // keep the next tile's loads ahead of this tile's waits (the scheduler
        // would otherwise sink them below them, leaving nothing in flight)
        __builtin_amdgcn_sched_barrier(0);
        const Tile& cur = ring[tt % (PF + 1)];
        const f32x4 Tcur = dot_q(cur.v);
        // coefficient product in fp32 (8 accumulating 16x16x4 steps per page at
        // rank 8): lane (w, c) element v holds T[page v/KS2][KS2 w + v%KS2][head c],
        // its B operand for k-step v%KS2 of page v/KS2
        f32x4 L[PPT][MT];
#pragma unroll
        for (int p = 0; p < PPT; ++p)
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                const float b = betas[tt * PPT + p];
                L[p][mt] = f32x4{b, b, b, b};
#pragma unroll
                for (int ks = 0; ks < KS2; ++ks)
                    L[p][mt] = mfma_16x16x4_f32(coef_el(cur, p, mt, ks), Tcur[p * KS2 + ks], L[p][mt]);
            }

#pragma unroll
        for (int p = 0; p < PPT; ++p) {
            const int pb = tt * PPT + p;
            page_mass_shifted<MT, kHeads, kMasked>(a, x, L[p], pb, page_shift(sv, pb), run_mx);
        }
        // a run ends with this tile: its maximum (row w holds pages 4w..4w+3)
        if ((tt + 1) * PPT % kRunPages == 0) {
            if (a.run_max) {
                const float rm = max_over_rows(run_mx);
                const int nruns = (a.max_pages + kRunPages - 1) / kRunPages;
                const int run = (x.j0 + tt * PPT) / kRunPages;
                if (x.lane == 0 && run < nruns)
                    a.run_max[((size_t)x.b * Hkv + g) * nruns + run] = rm;
            }
            run_mx = -INFINITY;
        }
    }
}

// bf16 summaries on the bf16 matrix cores, to fp32 accuracy: the stored
// values are bf16 already, and each fp32 multiplicand (q, and the basis
// product T) is split into three bf16 parts hi + mid + lo whose sum is the
// value (24 significant bits); every product is exact and accumulates in
// fp32.  Per tile of 16 basis rows (row m = basis row m % RR of page m / RR):
//   T (16 rows x 16 heads)   = basis rows . q^T   v_mfma_f32_16x16x32_bf16 x 3 parts per 32 d
//   L (16 tokens x 16 heads) = coef . T           v_mfma_f32_16x16x16_bf16 x 3 parts
// The coefficient operand of page p is zero outside p's rows of the tile.
__device__ __forceinline__ void split3(float x, __bf16& h, __bf16& m, __bf16& l) {
    h = (__bf16)x;
    float rest = x - (float)h;
    m = (__bf16)rest;
    rest -= (float)m;
    l = (__bf16)rest;
}

template <int P, int D, int RR, bool kExact, bool kHeads, bool kOff32, bool kMasked>
__device__ __forceinline__ void scan_batch_bf16(const ScanParams& a, const WaveCtx<D>& x) {
    using TS = uint16_t;
    constexpr int PPT = 16 / RR;          // pages per tile
    constexpr int NTILE = kBatch / PPT;
    constexpr int MT = P / 16;            // token tiles per page
    constexpr int NCH = D / 32;           // 32-wide d chunks (one 16-byte load per lane each)
    constexpr int WPP = RR / 4;           // lane groups per page in the coefficient operand
    constexpr int PF = kPrefetch;
    using Off = typename std::conditional<kOff32, uint32_t, size_t>::type;
    // the exact path's rank is the compile-time RR (address products become shifts)
    const int w = x.w, c = x.c, g = x.g, Hkv = x.Hkv, r = kExact ? RR : x.r;
    const int my_phys = x.my_phys;

    // q parts, in the order of the summary loads: chunk t holds d = 32t + 8w + e.
    // Split after the first tile's and the centroids' loads are issued.
    bf16x8 qp[3][NCH];
    auto split_q = [&]() {
        float qv[D / 4];
        query_after_loads<D / 4>(x.qf, qv);
#pragma unroll
        for (int t = 0; t < NCH; ++t)
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                __bf16 h, m, l;
                split3(qv[8 * t + e] * x.qs, h, m, l);
                qp[0][t][e] = h;
                qp[1][t][e] = m;
                qp[2][t][e] = l;
            }
    };

    const int a_pin = c / RR, a_k = c % RR;   // basis row loaded by this lane
    const int c_pin = w / WPP;                // page whose coefficients this lane supplies
    const int c_k0 = 4 * (w % WPP);           // its first coefficient index
    struct Tile {
        u32x4 v[NCH];
        u32x2 cf[MT];
    };
    auto load_tile = [&](int tt, Tile& T) {
        const int pj = __shfl(my_phys, tt * PPT + a_pin, kWave);
        const bool row_ok = !kMasked || (pj >= 0 && a_k < r);
        const Off src = (((Off)(kMasked && pj < 0 ? 0 : pj) * Hkv + g) * r +
                         (kMasked && a_k >= r ? r - 1 : a_k)) * D + 8 * w;
#pragma unroll
        for (int t = 0; t < NCH; ++t) {
            const u32x4 v = *reinterpret_cast<const u32x4*>(elem_addr<TS, kOff32>(a.basis, src + 32 * t));
#pragma unroll
            for (int e = 0; e < 4; ++e) T.v[t][e] = row_ok ? v[e] : 0u;
        }
        const int pp = __shfl(my_phys, tt * PPT + c_pin, kWave);
        const bool ok = !kMasked || pp >= 0;
        const Off csrc = ((Off)(kMasked && pp < 0 ? 0 : pp) * Hkv + g) * P * r;
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            const Off row = csrc + (Off)(16 * mt + c) * r;
            if constexpr (kExact) {
                const u32x2 v = *reinterpret_cast<const u32x2*>(elem_addr<TS, kOff32>(a.coef, row + c_k0));
                T.cf[mt][0] = ok ? v[0] : 0u;
                T.cf[mt][1] = ok ? v[1] : 0u;
            } else {  // padded rank: element by element, clamped and zeroed past it
                uint32_t hv[4];
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int kk = c_k0 + e;
                    const uint32_t h = *reinterpret_cast<const uint16_t*>(
                        elem_addr<TS, kOff32>(a.coef, row + (kk < r ? kk : r - 1)));
                    hv[e] = (ok && kk < r) ? h : 0u;
                }
                T.cf[mt][0] = hv[0] | (hv[1] << 16);
                T.cf[mt][1] = hv[2] | (hv[3] << 16);
            }
        }
    };

    Tile ring[PF + 1];
#pragma unroll
    for (int i = 0; i < PF && i < NTILE; ++i) load_tile(i, ring[i]);

    // beta tile: A row m = page j0 + m (lane column c supplies row c).
    f32x4 beta;
    {
        const Off src = ((Off)(my_phys < 0 ? 0 : my_phys) * Hkv + g) * D + 8 * w;
        f32x4 bacc[3];
#pragma unroll
        for (int i = 0; i < 3; ++i) bacc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
        u32x4 mv[NCH];
#pragma unroll
        for (int t = 0; t < NCH; ++t) {
            mv[t] = *reinterpret_cast<const u32x4*>(elem_addr<TS, kOff32>(a.mu, src + 32 * t));
        }
#pragma unroll
        for (int t = 0; t < NCH; ++t) {
            after_loads(mv[t]);
#pragma unroll
            for (int e = 0; e < 4; ++e) mv[t][e] = (!kMasked || my_phys >= 0) ? mv[t][e] : 0u;
        }
        split_q();
#pragma unroll
        for (int t = 0; t < NCH; ++t)
#pragma unroll
            for (int i = 0; i < 3; ++i) bacc[i] = mfma_16x16x32_bf16(as_bf16x8(mv[t]), qp[i][t], bacc[i]);
        beta = bacc[0] + bacc[1] + bacc[2];
    }
    // the coefficient products start from beta - shift (page_mass_shifted)
    float sv[1][4];
    float betas[kBatch];
    {
        __shared__ float tbl[4][16][kBatch];  // [wave of the block][head][page]
        shift_betas<1>(&beta, x.head_ok, w, c, tbl[threadIdx.x >> 6], betas, sv);
    }

    float run_mx = -INFINITY;
#pragma unroll
    for (int tt = 0; tt < NTILE; ++tt) {
        if (tt + PF < NTILE) load_tile(tt + PF, ring[(tt + PF) % (PF + 1)]);
        // keep the next tile's loads ahead of this tile's waits (the scheduler
        // would otherwise sink them below them, leaving nothing in flight)
        __builtin_amdgcn_sched_barrier(0);
        const Tile& cur = ring[tt % (PF + 1)];
        f32x4 tacc[3];
#pragma unroll
        for (int i = 0; i < 3; ++i) tacc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int t = 0; t < NCH; ++t)
#pragma unroll
            for (int i = 0; i < 3; ++i) tacc[i] = mfma_16x16x32_bf16(as_bf16x8(cur.v[t]), qp[i][t], tacc[i]);
        const f32x4 T = tacc[0] + tacc[1] + tacc[2];
        // lane (w, c) holds T[tile row 4w + v][head c]: its B operand rows of the
        // coefficient product, split into three bf16 parts
        bf16x4 tp[3];
        {
            __bf16 hv[4], mv[4], lv[4];
#pragma unroll
            for (int v = 0; v < 4; ++v) split3(T[v], hv[v], mv[v], lv[v]);
            typedef __bf16 bf16v4 __attribute__((ext_vector_type(4)));
            tp[0] = __builtin_bit_cast(bf16x4, bf16v4{hv[0], hv[1], hv[2], hv[3]});
            tp[1] = __builtin_bit_cast(bf16x4, bf16v4{mv[0], mv[1], mv[2], mv[3]});
            tp[2] = __builtin_bit_cast(bf16x4, bf16v4{lv[0], lv[1], lv[2], lv[3]});
        }
        f32x4 L[PPT][MT];
#pragma unroll
        for (int p = 0; p < PPT; ++p)
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                const bool mine = c_pin == p;
                const u32x2 av = {mine ? cur.cf[mt][0] : 0u, mine ? cur.cf[mt][1] : 0u};
                const bf16x4 A = as_bf16x4(av);
                const float b = betas[tt * PPT + p];
                f32x4 acc = mfma_16x16x16_bf16(A, tp[0], f32x4{b, b, b, b});
                acc = mfma_16x16x16_bf16(A, tp[1], acc);
                L[p][mt] = mfma_16x16x16_bf16(A, tp[2], acc);
            }
#pragma unroll
        for (int p = 0; p < PPT; ++p) {
            const int pb = tt * PPT + p;
            page_mass_shifted<MT, kHeads, kMasked>(a, x, L[p], pb, page_shift(sv, pb), run_mx);
        }
    }
    if (a.run_max && x.lane == 0) {
        const int nruns = (a.max_pages + kRunPages - 1) / kRunPages;
        a.run_max[((size_t)x.b * Hkv + g) * nruns + x.j0 / kBatch] = run_mx;
    }
}

// The KS2 int8 codes in the low bytes of v as floats, one sign-extending
// byte convert each (v a full word: nothing known about its upper bytes).
template <int KS2>
__device__ __forceinline__ void sbytes_f32(uint32_t v, float* out) {
#pragma unroll
    for (int k = 0; k < KS2; ++k) out[k] = (float)(int8_t)(v >> (8 * k));
}

// One batch of kBatch pages with integer-code summaries (int8 centroid and
// coefficients, int4 basis, one fp32 scale per vector).  With codes m, v, c
// and scales s_mu, s_v[k], s_c[k]:
//   beta = s_mu (m . q),   T_k = s_v[k] s_c[k] (v_k . q),   logit_i = beta + sum_k c_ik T_k,
// the estimator on the dequantised summary (scale * code).
//
// The query is held as four signed 8-bit digits per value: with E the
// exponent of head h's largest |q| (|q| < 2^E), X = trunc(q 2^(30-E)) =
// d0 + 2^8 d1 + 2^16 d2 + 2^24 d3, digits in [-128, 127], read off the bytes
// of (X + 0x808080) ^ 0x808080.  Code-by-digit products run on the int8
// matrix cores and are exact in int32; the four digit sums meet in fp32
// (relative error ~2^-24, that of fp32 arithmetic).  int4 basis codes c are
// widened to the bytes c + 8 (a few bit operations per 8 codes) and the +8
// comes off through the accumulator's starting value, -8 times the digits'
// sums over d (one int8 product with a ones matrix, once per wave).  The
// coefficient product runs in fp32 (16x16x4 steps) on codes converted one
// instruction each, from a starting value of beta, so the logits leave it
// with the centroid term in.
template <int P, int D, int RR, bool kExact, bool kHeads, bool kOff32, bool kMasked, int PF>
__device__ __forceinline__ void scan_batch_q(const ScanParams& a, const WaveCtx<D>& x) {
    constexpr int PPT = 16 / RR;          // pages per basis tile
    constexpr int NTILE = kBatch / PPT;
    constexpr int MT = P / 16;            // token tiles per page
    constexpr int KS2 = RR / 4;           // coefficient k-steps per page (codes per lane)
    constexpr int NW = D / 32;            // basis words (8 int4 codes) per lane and row
    constexpr int NCK = D / 64;           // 64-deep int8 products over d
    constexpr int NQ = D / 4;             // query values per lane
    static_assert(D % 64 == 0, "d a multiple of 64");
    static_assert(PF >= 1, "at least one tile in flight");
    using Off = typename std::conditional<kOff32, uint32_t, size_t>::type;
    // the exact path's rank is the compile-time RR (address products become shifts)
    const int w = x.w, c = x.c, g = x.g, Hkv = x.Hkv, r = kExact ? RR : x.r;
    const int my_phys = x.my_phys;
    const int SC = 1 + 2 * r;             // scales per unit
    const uint8_t* const mu_q = static_cast<const uint8_t*>(a.mu);
    const uint8_t* const basis_q = static_cast<const uint8_t*>(a.basis);
    const uint8_t* const coef_q = static_cast<const uint8_t*>(a.coef);
    // scales of the unit (block, g): 32-bit byte offsets when the arrays allow
    auto scales_of = [&](int blk) -> const float* {
        const Off o = ((Off)blk * Hkv + g) * SC;
        return reinterpret_cast<const float*>(reinterpret_cast<const char*>(a.scales) +
                                              (Off)(o * (Off)sizeof(float)));
    };

    // Basis row loaded by the lane (tile row m = c): page (m%4)/KS2 of the
    // tile, row KS2 (m/4) + (m%4)%KS2.  Row 4w + v of T is then page v / KS2,
    // k = KS2 w + v % KS2: the lane's B operand of k-step v % KS2 of that page.
    const int a_pin = (c & 3) / KS2;
    const int a_kk = KS2 * (c >> 2) + ((c & 3) % KS2);
    struct Tile {
        uint32_t v[NW];          // 8 int4 codes each, d = 32t + 8w + e
        uint32_t cf[PPT][MT];    // the aligned word holding codes k = KS2 w .. KS2 w + KS2 - 1
    };
    // the lane's codes start at bit cshift of its coefficient word (rank
    // RR: a token's row of r codes is word-aligned)
    const uint32_t cshift = kExact ? (uint32_t)(8 * ((KS2 * w) & 3)) : 0u;
    // Loaded words stay as they are until the tile is computed (arithmetic on
    // them here would wait for the next tile's loads right after issuing them).
    auto load_tile = [&](int tt, Tile& T) {
        const int pj = __shfl(my_phys, tt * PPT + a_pin, kWave);
        const bool row_ok = !kMasked || (pj >= 0 && a_kk < r);
        const Off src = (((Off)(kMasked && pj < 0 ? 0 : pj) * Hkv + g) * r +
                         (kMasked && a_kk >= r ? r - 1 : a_kk)) * (D / 2) + 4 * w;
#pragma unroll
        for (int t = 0; t < NW; ++t) {
            const uint32_t v = *reinterpret_cast<const uint32_t*>(basis_q + src + 16 * t);
            T.v[t] = row_ok ? v : 0u;
        }
#pragma unroll
        for (int p = 0; p < PPT; ++p) {
            const int pp = __builtin_amdgcn_readlane(my_phys, tt * PPT + p);
            const bool ok = !kMasked || pp >= 0;
            const Off csrc = ((Off)(kMasked && pp < 0 ? 0 : pp) * Hkv + g) * P * r;
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                const Off row = csrc + (Off)(16 * mt + c) * r;
                if constexpr (kExact) {
                    const uint32_t v =
                        *reinterpret_cast<const uint32_t*>(coef_q + row + ((KS2 * w) & ~3));
                    T.cf[p][mt] = ok ? v : 0u;
                } else {  // padded rank: byte by byte, clamped and zeroed past it
                    uint32_t hv = 0u;
#pragma unroll
                    for (int ks = 0; ks < KS2; ++ks) {
                        const int kk = KS2 * w + ks;
                        const uint32_t b = coef_q[row + (kk < r ? kk : r - 1)];
                        hv |= ((ok && kk < r) ? b : 0u) << (8 * ks);
                    }
                    T.cf[p][mt] = hv;
                }
            }
        }
    };

    // s_v[k] s_c[k] of every page and row of the batch: lane l loads page
    // l / 4, rows KS2 (l%4) .. + KS2 - 1 (0 past the rank or for an absent page)
    float sl_v[KS2], sl_c[KS2];
    {
        const int ps = __shfl(my_phys, x.lane >> 2, kWave);
        const float* sp = scales_of(ps < 0 ? 0 : ps);
#pragma unroll
        for (int e = 0; e < KS2; ++e) {
            const int k = KS2 * (x.lane & 3) + e;
            const int kc = kExact || k < r ? k : r - 1;
            sl_v[e] = sp[1 + kc];
            sl_c[e] = sp[1 + r + kc];
            if (ps < 0 || (!kExact && k >= r)) sl_v[e] = 0.0f;
        }
    }
    // centroid scales of pages j0 + 4w + v (the rows of the beta product this
    // lane receives)
    float smu[4];
#pragma unroll
    for (int v = 0; v < 4; ++v) {
        const int pv = __shfl(my_phys, 4 * w + v, kWave);
        smu[v] = pv < 0 ? 0.0f : scales_of(pv)[0];
    }
    // centroid codes of page j0 + c (row c of the beta product), d = 32t + 8w + e
    u32x2 m8[NW];
    {
        const Off src = ((Off)(my_phys < 0 ? 0 : my_phys) * Hkv + g) * D + 8 * w;
#pragma unroll
        for (int t = 0; t < NW; ++t) m8[t] = *reinterpret_cast<const u32x2*>(mu_q + src + 32 * t);
    }
    // the first tiles' loads follow the ones the batch's set-up waits for
    Tile ring[PF + 1];
#pragma unroll
    for (int i = 0; i < PF && i < NTILE; ++i) load_tile(i, ring[i]);

    // Query digits.  Word wd of product chunk j holds d = 32t + 8w + pi + 2k in
    // byte k, t = 2j + wd/2, pi = wd%2: even d of a basis word's 8, then odd.
    i32x4 qd[4][NCK];
    float p2;  // 2^(E-30): the digits' unit
    {
        float qv[NQ];
        query_after_loads<NQ>(x.qf, qv);
        float amax = 0.0f;
#pragma unroll
        for (int i = 0; i < NQ; ++i) {
            qv[i] *= x.qs;
            amax = fmaxf(amax, fabsf(qv[i]));
        }
        amax = max_over_rows(amax);
        int E = __builtin_amdgcn_frexp_expf(amax);  // amax < 2^E; 0 for amax 0
        E = E < -90 ? -90 : (E > 120 ? 120 : E);
        const float up = __builtin_ldexpf(1.0f, 30 - E);
        p2 = __builtin_ldexpf(1.0f, E - 30);
#pragma unroll
        for (int t = 0; t < NW; ++t)
#pragma unroll
            for (int pi = 0; pi < 2; ++pi) {
                uint32_t z[4];
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    const int X = (int)(qv[8 * t + pi + 2 * k] * up);
                    z[k] = ((uint32_t)X + 0x808080u) ^ 0x808080u;
                }
                // 4 x 4 byte transpose: digit i of the four values
                const uint32_t lo_ab = __builtin_amdgcn_perm(z[1], z[0], 0x05010400u);
                const uint32_t hi_ab = __builtin_amdgcn_perm(z[1], z[0], 0x07030602u);
                const uint32_t lo_cd = __builtin_amdgcn_perm(z[3], z[2], 0x05010400u);
                const uint32_t hi_cd = __builtin_amdgcn_perm(z[3], z[2], 0x07030602u);
                const int j = t / 2, wd = 2 * (t % 2) + pi;
                qd[0][j][wd] = (int)__builtin_amdgcn_perm(lo_cd, lo_ab, 0x05040100u);
                qd[1][j][wd] = (int)__builtin_amdgcn_perm(lo_cd, lo_ab, 0x07060302u);
                qd[2][j][wd] = (int)__builtin_amdgcn_perm(hi_cd, hi_ab, 0x05040100u);
                qd[3][j][wd] = (int)__builtin_amdgcn_perm(hi_cd, hi_ab, 0x07060302u);
            }
    }
    // starting values of the basis product: -8 times each digit's sum over d,
    // digits 0 and 1 (and 2 and 3) in the accumulator the pair combines into
    int bias_lo, bias_hi;
    {
        const i32x4 ones = {0x01010101, 0x01010101, 0x01010101, 0x01010101};
        i32x4 S[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            S[i] = i32x4{0, 0, 0, 0};
#pragma unroll
            for (int j = 0; j < NCK; ++j) S[i] = mfma_16x16x64_i8(ones, qd[i][j], S[i]);
        }
        bias_lo = (int)(0u - 8u * ((uint32_t)S[0][0] + 256u * (uint32_t)S[1][0]));
        bias_hi = (int)(0u - 8u * ((uint32_t)S[2][0] + 256u * (uint32_t)S[3][0]));
    }
    // digit sums -> fp32 in units of the digits (times p2 for q's units)
    auto combine = [](const i32x4* acc, int v) -> float {
        const int r10 = (int)(((uint32_t)acc[1][v] << 8) + (uint32_t)acc[0][v]);
        const int r32 = (int)(((uint32_t)acc[3][v] << 8) + (uint32_t)acc[2][v]);
        return fmaf((float)r32, 65536.0f, (float)r10);
    };

    // beta - shift of the batch's 16 pages for the lane's head, in every lane:
    // the product gives lane (w, c) pages 4w..4w+3; a per-wave table in LDS
    // hands each lane the other twelve.  shift of page 4w + v = the largest
    // beta over the group's heads, in sv[0][v] of lane (w, c).
    float betas[kBatch];
    float sv[1][4];
    __shared__ float stbl[4][kBatch][RR];     // [wave of the block][page][row]: s_v s_c
    const int wv = threadIdx.x >> 6;
    {
        __shared__ float tbl[4][16][kBatch];  // [wave of the block][head][page]
        i32x4 acc[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[i] = i32x4{0, 0, 0, 0};
#pragma unroll
        for (int t = 0; t < NW; ++t) {
            after_loads(m8[t]);
            if (kMasked && my_phys < 0) m8[t] = u32x2{0u, 0u};
        }
#pragma unroll
        for (int j = 0; j < NCK; ++j) {
            const i32x4 mw = {(int)__builtin_amdgcn_perm(m8[2 * j][1], m8[2 * j][0], 0x06040200u),
                              (int)__builtin_amdgcn_perm(m8[2 * j][1], m8[2 * j][0], 0x07050301u),
                              (int)__builtin_amdgcn_perm(m8[2 * j + 1][1], m8[2 * j + 1][0], 0x06040200u),
                              (int)__builtin_amdgcn_perm(m8[2 * j + 1][1], m8[2 * j + 1][0], 0x07050301u)};
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[i] = mfma_16x16x64_i8(mw, qd[i][j], acc[i]);
        }
        f32x4 bt;
#pragma unroll
        for (int v = 0; v < 4; ++v) bt[v] = combine(acc, v) * p2 * smu[v];
#pragma unroll
        for (int e = 0; e < KS2; ++e) stbl[wv][x.lane >> 2][KS2 * (x.lane & 3) + e] = sl_v[e] * sl_c[e];
        // (the helper's wait for its LDS writes covers these too)
        shift_betas<1>(&bt, x.head_ok, w, c, tbl[wv], betas, sv);
    }

    // Products of tile tt (matrix cores) are issued before the page masses of
    // tile tt - 1 (VALU), so the two overlap.
    auto products = [&](int tt, const Tile& cur, f32x4 (*L)[MT]) {
        // T (16 rows x 16 heads) on the int8 matrix cores, one accumulator per digit
        i32x4 acc[4] = {i32x4{bias_lo, bias_lo, bias_lo, bias_lo}, i32x4{0, 0, 0, 0},
                        i32x4{bias_hi, bias_hi, bias_hi, bias_hi}, i32x4{0, 0, 0, 0}};
#pragma unroll
        for (int j = 0; j < NCK; ++j) {
            const uint32_t u0 = cur.v[2 * j] ^ 0x88888888u, u1 = cur.v[2 * j + 1] ^ 0x88888888u;
            const i32x4 bw = {(int)(u0 & 0x0F0F0F0Fu), (int)((u0 >> 4) & 0x0F0F0F0Fu),
                              (int)(u1 & 0x0F0F0F0Fu), (int)((u1 >> 4) & 0x0F0F0F0Fu)};
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[i] = mfma_16x16x64_i8(bw, qd[i][j], acc[i]);
        }
        // row 4w + v of T: page tt PPT + v / KS2, k = KS2 w + v % KS2
        float T[4];
#pragma unroll
        for (int v = 0; v < 4; ++v)
            T[v] = combine(acc, v) * p2 * stbl[wv][tt * PPT + v / KS2][KS2 * w + v % KS2];
        // coefficient product in fp32 from beta: page p, k-step ks takes the
        // lane's code KS2 w + ks against T[KS2 p + ks]
#pragma unroll
        for (int p = 0; p < PPT; ++p)
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) {
                const float b = betas[tt * PPT + p];
                f32x4 l = {b, b, b, b};
                float cv[4];
                sbytes_f32<KS2>(cur.cf[p][mt] >> cshift, cv);
#pragma unroll
                for (int ks = 0; ks < KS2; ++ks) l = mfma_16x16x4_f32(cv[ks], T[KS2 * p + ks], l);
                L[p][mt] = l;
            }
    };
    float run_mx = -INFINITY;
    auto masses = [&](int tt, const f32x4 (*L)[MT]) {
#pragma unroll
        for (int p = 0; p < PPT; ++p) {
            const int pb = tt * PPT + p;
            page_mass_shifted<MT, kHeads, kMasked>(a, x, L[p], pb, page_shift(sv, pb), run_mx);
        }
    };
    f32x4 Lb[2][PPT][MT];
#pragma unroll
    for (int tt = 0; tt < NTILE; ++tt) {
        if (tt + PF < NTILE) load_tile(tt + PF, ring[(tt + PF) % (PF + 1)]);
        // keep the next tile's loads ahead of this tile's waits
        __builtin_amdgcn_sched_barrier(0);
        products(tt, ring[tt % (PF + 1)], Lb[tt & 1]);
        if (tt > 0) masses(tt - 1, Lb[(tt - 1) & 1]);
    }
    masses(NTILE - 1, Lb[(NTILE - 1) & 1]);
    if (a.run_max && x.lane == 0) {
        const int nruns = (a.max_pages + kRunPages - 1) / kRunPages;
        a.run_max[((size_t)x.b * Hkv + g) * nruns + x.j0 / kBatch] = run_mx;
    }
}

template <typename TS, int P, int D, int RR, bool kExact, bool kHeads, bool kOff32,
          int NP = kBatch, int PF = kPrefetch>
__global__ __launch_bounds__(256) void scan_kernel(const ScanParams a) {
    static_assert(P % 16 == 0 && D % 32 == 0, "P a multiple of 16, d of 32");
    static_assert(RR == 4 || RR == 8 || RR == 16, "padded rank");
    static_assert(NP % kRunPages == 0 && NP <= kWave, "whole runs per wave");
    static_assert(sizeof(TS) == 4 || NP == kBatch, "the bf16 and code paths scan one run per wave");
    static_assert(sizeof(TS) != 2 || PF == kPrefetch, "the bf16 path keeps one tile in flight");
    constexpr int E = Summ<TS>::E;
    constexpr int NCH = D / (4 * E);

    WaveCtx<D> x;
    x.lane = threadIdx.x & 63;
    x.w = x.lane >> 4;
    x.c = x.lane & 15;
    const int wave = blockIdx.x * 4 + (threadIdx.x >> 6);
    const int nbatch = (a.max_pages + NP - 1) / NP;
    if (wave >= a.batch * a.num_kv_heads * nbatch) return;
    const int jb = wave % nbatch;
    x.g = (wave / nbatch) % a.num_kv_heads;
    x.b = wave / (nbatch * a.num_kv_heads);
    x.Hkv = a.num_kv_heads;
    x.G = a.num_q_heads / x.Hkv;
    x.r = a.rank;
    x.head_ok = x.c < x.G;
    x.j0 = jb * NP;
    const int c = x.c, w = x.w;

    // Query fragment, in the contraction order of the summary loads:
    // qf[E t + e] = q[h][4E t + E w + e] for head h = c, as loaded; the batch
    // functions scale it to log2 units (qs, 0 for padding heads) when they
    // split it, after their first summary loads are issued.  Its loads go out
    // first: they depend on nothing the block table gives.
    x.qs = x.head_ok ? kLog2e / sqrtf((float)D) : 0.0f;
    {
        const float* qp =
            a.q + ((size_t)x.b * a.num_q_heads + x.g * x.G + (x.head_ok ? c : 0)) * D;
#pragma unroll
        for (int t = 0; t < NCH; ++t)
#pragma unroll
            for (int h4 = 0; h4 < E / 4; ++h4) {
                const f32x4 v = *reinterpret_cast<const f32x4*>(qp + 4 * E * t + E * w + 4 * h4);
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    x.qf[E * t + 4 * h4 + e] = v[e];
            }
    }

    // Lane l looks after page j0 + l % NP.  Its block-table entry is read
    // together with the sequence length (clamped index, kept only if the page
    // is full), so the two loads overlap instead of following each other.
    const int pl = x.lane % NP;
    const int jc = x.j0 + pl;
    const int p_spec =
        a.block_table[(size_t)x.b * a.max_pages + (jc < a.max_pages ? jc : a.max_pages - 1)];
    // the pages that compete: full pages whose summaries exist (the count is
    // read beside the length; pages past it are not scanned and get -inf)
    const int summ_raw = a.summarized ? a.summarized[x.b] : 0;
    const int full =
        candidate_pages(a.seq_lens[x.b], summ_raw, a.summarized != nullptr, P, a.max_pages);
    x.out_page = a.page_logmass + ((size_t)x.b * x.Hkv + x.g) * a.max_pages;
    if (x.j0 >= full) {  // whole batch past the full pages
        const int nruns = (a.max_pages + kRunPages - 1) / kRunPages;
        const int run = x.j0 / kRunPages + x.lane;
        if (a.run_max && x.lane < NP / kRunPages && run < nruns)
            a.run_max[((size_t)x.b * x.Hkv + x.g) * nruns + run] = -INFINITY;
        if (x.lane < NP && x.j0 + x.lane < a.max_pages) {
            x.out_page[x.j0 + x.lane] = -INFINITY;
            if constexpr (kHeads)
                for (int hh = 0; hh < x.G; ++hh)
                    a.head_logmass[((size_t)x.b * a.num_q_heads + x.g * x.G + hh) * a.max_pages +
                                   x.j0 + x.lane] = -INFINITY;
        }
        return;
    }
    x.my_phys = (jc < full && p_spec >= 0 && p_spec < a.num_blocks) ? p_spec : -1;


    // every page of the batch present and the rank not padded: no masking
    if constexpr (kExact) {
        if (x.j0 + NP <= full && __ballot(x.lane < NP && x.my_phys < 0) == 0ull) {
            if constexpr (sizeof(TS) == 1)
                scan_batch_q<P, D, RR, kExact, kHeads, kOff32, false, PF>(a, x);
            else if constexpr (sizeof(TS) == 2)
                scan_batch_bf16<P, D, RR, kExact, kHeads, kOff32, false>(a, x);
            else
                scan_batch_f32<P, D, RR, kExact, kHeads, kOff32, false, NP, PF>(a, x);
            return;
        }
    }
    if constexpr (sizeof(TS) == 1)
        scan_batch_q<P, D, RR, kExact, kHeads, kOff32, true, PF>(a, x);
    else if constexpr (sizeof(TS) == 2)
        scan_batch_bf16<P, D, RR, kExact, kHeads, kOff32, true>(a, x);
    else
        scan_batch_f32<P, D, RR, kExact, kHeads, kOff32, true, NP, PF>(a, x);
}

template <typename TS, int P, int D, int RR, bool kHeads, bool kOff32, int NP, int PF>
hipError_t launch4(const ScanParams& p, hipStream_t s) {
    const long waves = (long)p.batch * p.num_kv_heads * ((p.max_pages + NP - 1) / NP);
    const unsigned blocks = (unsigned)((waves + 3) / 4);
    if (blocks == 0) return hipSuccess;
    if (p.rank == RR)
        hipLaunchKernelGGL((scan_kernel<TS, P, D, RR, true, kHeads, kOff32, NP, PF>),
                           dim3(blocks), dim3(256), 0, s, p);
    else
        hipLaunchKernelGGL((scan_kernel<TS, P, D, RR, false, kHeads, kOff32, NP, PF>),
                           dim3(blocks), dim3(256), 0, s, p);
    return hipGetLastError();
}

template <typename TS, int P, int D, int RR, int NP = kBatch, int PF = kPrefetch>
hipError_t launch_ts(const ScanParams& p, hipStream_t s) {
    // largest summary array (basis or coefficients) in bytes
    size_t per_unit = (size_t)p.rank * (D > P ? D : P) * sizeof(TS);
    if (sizeof(TS) == 1) {  // codes: centroid D, basis r D/2, coefficients P r bytes
        per_unit = (size_t)p.rank * (D / 2 > P ? D / 2 : P);
        per_unit = per_unit > (size_t)D ? per_unit : (size_t)D;
    }
    const bool off32 = (size_t)p.num_blocks * p.num_kv_heads * per_unit < (size_t(1) << 32);
    if (p.head_logmass != nullptr)
        return off32 ? launch4<TS, P, D, RR, true, true, NP, PF>(p, s)
                     : launch4<TS, P, D, RR, true, false, NP, PF>(p, s);
    return off32 ? launch4<TS, P, D, RR, false, true, NP, PF>(p, s)
                 : launch4<TS, P, D, RR, false, false, NP, PF>(p, s);
}

template <typename TS, int P, int D, int RR>
hipError_t launch_typed(const ScanParams& p, hipStream_t s) {
    if constexpr (sizeof(TS) == 1)
        return launch_ts<TS, P, D, RR, kBatch, kCodePrefetch>(p, s);
    else
        return launch_ts<TS, P, D, RR>(p, s);
}

template <typename TS, int P, int D>
hipError_t launch_rr(const ScanParams& p, hipStream_t s) {
    if (p.rank <= 4) return launch_typed<TS, P, D, 4>(p, s);
    if (p.rank <= 8) return launch_typed<TS, P, D, 8>(p, s);
    return launch_typed<TS, P, D, 16>(p, s);
}

// Every supported (page size, head dim) for one stored summary type.
template <typename TS>
hipError_t launch_scan_of(const ScanParams& p, hipStream_t s) {
    if (p.page_size == 16 && p.head_dim == 64) return launch_rr<TS, 16, 64>(p, s);
    if (p.page_size == 16 && p.head_dim == 128) return launch_rr<TS, 16, 128>(p, s);
    if (p.page_size == 64 && p.head_dim == 64) return launch_rr<TS, 64, 64>(p, s);
    return launch_rr<TS, 64, 128>(p, s);
}

}  // namespace

}  // namespace locks
