// Summary scan, fp32 summaries: one wave's batch of pages.
#pragma once

#include "scan_common.hpp"

namespace locks {

namespace {

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

}  // namespace

}  // namespace locks
