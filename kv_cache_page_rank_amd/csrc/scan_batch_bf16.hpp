// Summary scan, bf16 summaries: one wave's batch of pages.
#pragma once

#include "scan_common.hpp"

namespace locks {

namespace {

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

}  // namespace

}  // namespace locks
