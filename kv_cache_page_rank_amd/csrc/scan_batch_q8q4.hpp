// Summary scan, int8 / int4 code summaries: one wave's batch of pages.
#pragma once

#include "scan_common.hpp"

namespace locks {

namespace {

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
// Per-workgroup LDS tables of the code path (one set for the masked and the
// unmasked batch of a kernel): per wave, s_v s_c of each page and row, beta -
// shift of each head and page, and the query digits of each lane.
template <int RR, int NCK>
struct CodeLds {
    float scale[4][kBatch][RR];
    float beta[4][16][kBatch];
    i32x4 qd[4][4][NCK][64];
};
template <int RR, int NCK>
__device__ __forceinline__ CodeLds<RR, NCK>& code_lds() {
    __shared__ CodeLds<RR, NCK> lds;
    return lds;
}

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

    // beta - shift of the batch's 16 pages for each head: the product gives
    // lane (w, c) pages 4w..4w+3; they go to the per-wave LDS table, where
    // every lane reads its head's entry of each page as the page comes up.
    // shift of page 4w + v = the largest beta over the group's heads, in
    // sv[0][v] of lane (w, c).  The query digits move to LDS as well (the
    // tiles read them back), which keeps the kernel within three waves'
    // registers per SIMD.
    float sv[1][4];
    CodeLds<RR, NCK>& lds = code_lds<RR, NCK>();
    auto& stbl = lds.scale;  // [wave of the block][page][row]: s_v s_c
    auto& tbl = lds.beta;    // [wave of the block][head][page]: beta - shift
    auto& qtbl = lds.qd;     // [wave][digit][chunk][lane]: the query digits
    const int wv = threadIdx.x >> 6;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < NCK; ++j) qtbl[wv][i][j][x.lane] = qd[i][j];
    {
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
        shift_betas<1>(&bt, x.head_ok, w, c, tbl[wv], nullptr, sv);
    }

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
            for (int i = 0; i < 4; ++i) acc[i] = mfma_16x16x64_i8(bw, qtbl[wv][i][j][x.lane], acc[i]);
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
                const float b = tbl[wv][c][tt * PPT + p];
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
#pragma unroll
    for (int tt = 0; tt < NTILE; ++tt) {
        // When the whole launch is resident at once, a wave's issue priority
        // falls as it advances, so the waves sharing a SIMD progress together
        // instead of the older one finishing first and the younger one
        // running its last tiles alone (measured: 21.3 -> 20.8 us at 1M
        // tokens; with several rounds of waves it slows the scan, as the
        // waves starting later take the issue slots).
        if (a.one_round) {
            constexpr int kLevels = 4;
            const int pr = kLevels - 1 - (kLevels * tt) / NTILE;  // constant once unrolled
            if (pr == 3)
                __builtin_amdgcn_s_setprio(3);
            else if (pr == 2)
                __builtin_amdgcn_s_setprio(2);
            else if (pr == 1)
                __builtin_amdgcn_s_setprio(1);
            else
                __builtin_amdgcn_s_setprio(0);
        }
        if (tt + PF < NTILE) load_tile(tt + PF, ring[(tt + PF) % (PF + 1)]);
        // keep the next tile's loads ahead of this tile's waits
        __builtin_amdgcn_sched_barrier(0);
        f32x4 Lc[PPT][MT];
        products(tt, ring[tt % (PF + 1)], Lc);
        masses(tt, Lc);
    }
    if (a.run_max && x.lane == 0) {
        const int nruns = (a.max_pages + kRunPages - 1) / kRunPages;
        a.run_max[((size_t)x.b * Hkv + g) * nruns + x.j0 / kBatch] = run_mx;
    }
}

}  // namespace

}  // namespace locks
