// Shared pieces of the summary-scan kernels (scan_kernel.hpp assembles the
// kernel from scan_batch_f32.hpp, scan_batch_bf16.hpp and
// scan_batch_q8q4.hpp, one per stored summary type).
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
constexpr int kPrefetch = 1;       // their tiles in flight ahead
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
// for its head in betas[] (null: it reads them from the table later), through
// a per-wave LDS table tbl[16][16 NR], and lane (w, c) keeps the shifts of
// pages 16n + 4w + v in sv[n][v].
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
    if (betas == nullptr) return;  // the caller reads the table itself
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

}  // namespace

}  // namespace locks
