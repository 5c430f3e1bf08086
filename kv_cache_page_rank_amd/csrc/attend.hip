// Split-K paged flash-decode over a page list, and the log-sum-exp merge.
//
// Sparse: for each (b, g) one split per selected page plus one tail split for
// every page without a summary (abstract: only the top pages are attended; a
// page's summary is made once the page is final, so the partial last page,
// and full pages whose summaries are still being built, are always
// attended): pages [cand, n_all), where cand = min(summarised pages, full
// pages) - normally just the partial page.  Dense: each split is a run of
// consecutive pages (the dense-attention baseline).
// A split emits, per query head, the running max m and sum l (log2 units)
// and the unnormalised output o; the merge combines the splits of a head in
// split order: M = max m_s, L = sum l_s 2^(m_s - M), out = sum o_s 2^(m_s - M) / L,
// lse = (M + log2 L) ln 2.
//
// bf16 caches (P = 64): MFMA for both products with the group's (up to 16)
// heads as the 16-wide MFMA dimension; q is split into three bf16 parts
// (~24 significant bits) and p into two (~16).  V pages are stored
// transposed ([d][P]) so that each lane's contraction elements (tokens) are
// contiguous.
#include "device_common.hpp"
#include "launchers.hpp"

namespace locks {

namespace {

struct SplitPages {
    int first, count;  // consecutive logical pages [first, first + count)
};

// Candidates of sequence b (full pages with summaries; attention needs the
// count to know which pages the tail split covers).
__device__ __forceinline__ int attn_candidates(const AttnParams& a, int b, int seq_raw) {
    return candidate_pages(seq_raw, a.summarized ? a.summarized[b] : 0, a.summarized != nullptr,
                           a.page_size, a.max_pages);
}

__device__ __forceinline__ SplitPages split_pages(const AttnParams& a, bool sparse, int b, int g,
                                                  int s, int cand, int n_all) {
    SplitPages r{0, 0};
    if (sparse) {
        if (s < a.k_sel) {
            const int j = a.sel_pages[((size_t)b * a.num_kv_heads + g) * a.k_sel + s];
            if (j >= 0 && j < cand) r = {j, 1};
        } else if (n_all > cand) {
            r = {cand, n_all - cand};  // pages without a summary (the tail)
        }
    } else {
        const int lo = s * a.pages_per_split;
        const int hi = lo + a.pages_per_split < n_all ? lo + a.pages_per_split : n_all;
        if (lo < hi) r = {lo, hi - lo};
    }
    return r;
}

// Combine the (m, l, o) partials of the 4 waves of a workgroup (4
// consecutive splits of one (b, g)) into one partial, in wave order.
// sm_o[w][h][d]; thread t combines head t/16, dims [8*(t%16), +8).
template <int D>
__device__ __forceinline__ void combine_waves(const AttnParams& a, float (*sm_m)[16],
                                              float (*sm_l)[16], float (*sm_o)[16][D + 4], int b,
                                              int g, int G, int part, int nparts) {
    const int t = threadIdx.x;
    const int h = t >> 4;
    constexpr int DPT = D / 16;  // dims per thread
    const int d0 = (t & 15) * DPT;
    if (h >= G) return;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < 4; ++w)
        if (sm_l[w][h] > 0.f) M = fmaxf(M, sm_m[w][h]);
    float L = 0.f, o[DPT];
#pragma unroll
    for (int e = 0; e < DPT; ++e) o[e] = 0.f;
    if (M != -INFINITY) {
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            const float l = sm_l[w][h];
            const float wt = l > 0.f ? fast_exp2(sm_m[w][h] - M) : 0.f;
            L += l * wt;
#pragma unroll
            for (int e = 0; e < DPT; ++e) o[e] += sm_o[w][h][d0 + e] * wt;
        }
    }
    const size_t row = ((size_t)b * a.num_q_heads + g * G + h) * nparts + part;
    if ((t & 15) == 0) {
        a.part_ml[2 * row] = M;
        a.part_ml[2 * row + 1] = L;
    }
    float* dst = a.part_o + row * D + d0;
#pragma unroll
    for (int e = 0; e < DPT; e += 4)
        *reinterpret_cast<f32x4*>(dst + e) = f32x4{o[e], o[e + 1], o[e + 2], o[e + 3]};
}

// One wave per split (sparse: one selected page or the partial page; dense:
// a run of pages); the 4 waves of a workgroup take 4 consecutive splits of
// one (b, g) and are combined in LDS into one partial.  Per page and wave,
// with the group's heads as the 16-wide MFMA dimension:
//   S^T (64 tok x 16 h) = K (64 x d) . q^T   v_mfma_f32_16x16x32_bf16 (q in three parts)
//   O^T (d x 16 h)     += V^T (d x 64) . p^T v_mfma_f32_16x16x32_bf16 (p as hi + lo)
// All of a page's K and V fragments (32 KB per wave) are requested before
// any is used.  The token order inside the score tiles is chosen so that
// each lane's scores are exactly its 8 contraction elements of the value
// product: score tile mt, A row m  <->  token 32*(mt/2) + 8*(m/4) + 4*(mt%2) + m%4,
// and the value operand is 8 consecutive tokens of one V^T row (16 bytes).
// K and V fragments of one page for one wave (32 KB in 64 VGPRs x 2).
template <int P, int D>
struct PageFrag {
    static constexpr int KS = D / 32, MT = P / 16, KS2 = P / 32, MD = D / 16;
    u32x4 k[MT][KS];
    u32x4 v[KS2][MD];
};

// The query's three bf16 parts per 32-wide chunk: q = hi + mid + lo, each the
// nearest-even bf16 of what the previous parts leave (~24 significant bits),
// so a score from bf16 keys carries fp32-level error whatever its size.
template <int KS>
struct QParts {
    bf16x8 part[3][KS];
};

// Buffer descriptor of one page of `bytes` bytes at `base`; with `present`
// false it holds no records, so every load through it fetches nothing and
// returns zeros.  Loads through such descriptors can be issued
// unconditionally, which keeps the compiler's wait counts exact: after a
// branch that issues loads on one side only, its waits must hold for both
// sides and so also wait for loads that are not needed yet.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t page_rsrc(const void* base, bool present,
                                                            int bytes) {
    constexpr int kRawWord3 = 0x00020000;  // gfx9 family: 32-bit data format, raw access
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, present ? bytes : 0,
                                             kRawWord3);
}
// Keys of a page for one wave: score tile mt, A row m <-> token
// 32(mt/2) + 8(m/4) + 4(mt%2) + m%4; 16 bytes of d per load (byte offsets
// within the page).
template <int P, int D>
__device__ __forceinline__ void load_page_k_rsrc(__amdgpu_buffer_rsrc_t rs, int w, int c,
                                                 PageFrag<P, D>& f) {
    using F = PageFrag<P, D>;
#pragma unroll
    for (int mt = 0; mt < F::MT; ++mt) {
        const int tok = 32 * (mt >> 1) + 8 * (c >> 2) + 4 * (mt & 1) + (c & 3);
#pragma unroll
        for (int ks = 0; ks < F::KS; ++ks)
            f.k[mt][ks] = __builtin_bit_cast(
                u32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, 2 * (tok * D + 32 * ks + 8 * w), 0, 0));
    }
}

// Values of a page (stored [d][P]) for one wave: 8 consecutive tokens of one
// V^T row per 16-byte load.
template <int P, int D>
__device__ __forceinline__ void load_page_v_rsrc(__amdgpu_buffer_rsrc_t rs, int w, int c,
                                                 PageFrag<P, D>& f) {
    using F = PageFrag<P, D>;
#pragma unroll
    for (int ks2 = 0; ks2 < F::KS2; ++ks2)
#pragma unroll
        for (int md = 0; md < F::MD; ++md)
            f.v[ks2][md] = __builtin_bit_cast(
                u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                           rs, 2 * ((16 * md + c) * P + 32 * ks2 + 8 * w), 0, 0));
}

// Scores of one page (log2 units), tokens past nv set to -inf.
template <int P, int D>
__device__ __forceinline__ void page_scores(const PageFrag<P, D>& f, int nv, int w,
                                            const QParts<D / 32>& q, f32x4* sc) {
    using F = PageFrag<P, D>;
#pragma unroll
    for (int mt = 0; mt < F::MT; ++mt) {
        sc[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < F::KS; ++ks) {
            const bf16x8 kf = as_bf16x8(f.k[mt][ks]);
            sc[mt] = mfma_16x16x32_bf16(kf, q.part[2][ks], sc[mt]);
            sc[mt] = mfma_16x16x32_bf16(kf, q.part[1][ks], sc[mt]);
            sc[mt] = mfma_16x16x32_bf16(kf, q.part[0][ks], sc[mt]);
        }
    }
    // lane (w, c) element v of tile mt: token 32(mt/2) + 8w + 4(mt%2) + v, head c
    if (nv < P) {
#pragma unroll
        for (int mt = 0; mt < F::MT; ++mt)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int tok = 32 * (mt >> 1) + 8 * w + 4 * (mt & 1) + v;
                sc[mt][v] = tok < nv ? sc[mt][v] : -INFINITY;
            }
    }
}

// Online-softmax update of one wave's (m, l, O^T) with the scores of a page
// and its values.
template <int P, int D>
__device__ __forceinline__ void page_values(const PageFrag<P, D>& f, f32x4* sc, int nv, int w,
                                            float& m_run, float& l_run, f32x4* acc) {
    using F = PageFrag<P, D>;
    float mx = -INFINITY;
#pragma unroll
    for (int mt = 0; mt < F::MT; ++mt)
#pragma unroll
        for (int v = 0; v < 4; ++v) mx = fmaxf(mx, sc[mt][v]);
    mx = max_over_rows(mx);
    const float m_new = fmaxf(m_run, mx);
    if (m_new == -INFINITY) return;
    const float alpha = fast_exp2(m_run - m_new);
    float psum = 0.f;
#pragma unroll
    for (int mt = 0; mt < F::MT; ++mt)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            sc[mt][v] = fast_exp2(sc[mt][v] - m_new);
            psum += sc[mt][v];
        }
    l_run = l_run * alpha + psum;
    m_run = m_new;
#pragma unroll
    for (int md = 0; md < F::MD; ++md) acc[md] *= alpha;

#pragma unroll
    for (int ks2 = 0; ks2 < F::KS2; ++ks2) {
        // p operand: slot e2 = 4e + v <-> token 32ks2 + 8w + e2 <-> tile 2ks2 + e, element v
        u32x4 phi, plo;
#pragma unroll
        for (int e2 = 0; e2 < 4; ++e2) {
            const float p0 = sc[2 * ks2 + (e2 >> 1)][(2 * e2) & 3];
            const float p1 = sc[2 * ks2 + (e2 >> 1)][(2 * e2 + 1) & 3];
            uint16_t h0, l0, h1, l1;
            split_bf16(p0, h0, l0);
            split_bf16(p1, h1, l1);
            phi[e2] = (uint32_t)h0 | ((uint32_t)h1 << 16);
            plo[e2] = (uint32_t)l0 | ((uint32_t)l1 << 16);
        }
        const bf16x8 bhi = as_bf16x8(phi), blo = as_bf16x8(plo);
#pragma unroll
        for (int md = 0; md < F::MD; ++md) {
            u32x4 vr = f.v[ks2][md];
            if (nv < P) {  // zero values of absent tokens (their p is 0, their bits may be NaN)
#pragma unroll
                for (int e2 = 0; e2 < 4; ++e2) {
                    const int tok = 32 * ks2 + 8 * w + 2 * e2;
                    vr[e2] &= (tok < nv ? 0x0000ffffu : 0u) | (tok + 1 < nv ? 0xffff0000u : 0u);
                }
            }
            const bf16x8 vf = as_bf16x8(vr);
            acc[md] = mfma_16x16x32_bf16(vf, bhi, acc[md]);
            acc[md] = mfma_16x16x32_bf16(vf, blo, acc[md]);
        }
    }
}

// q fragment of head hq: the raw loads (q[hq][32ks + 8w + e], every chunk's
// loads in flight together) and their split into three bf16 parts in log2 units
// (zero for padding heads).
template <int D>
__device__ __forceinline__ void load_q_raw(const AttnParams& a, int b, int hq, int w, f32x4* xa,
                                           f32x4* xb) {
    const float* qp = a.q + ((size_t)b * a.num_q_heads + hq) * D;
#pragma unroll
    for (int ks = 0; ks < D / 32; ++ks) {
        xa[ks] = *reinterpret_cast<const f32x4*>(qp + 32 * ks + 8 * w);
        xb[ks] = *reinterpret_cast<const f32x4*>(qp + 32 * ks + 8 * w + 4);
    }
}
__device__ __forceinline__ void split3_bits(float x, uint16_t& h, uint16_t& m, uint16_t& l) {
    h = bf16_rne(x);
    const float r = x - bf16_bits_to_f32(h);
    m = bf16_rne(r);
    l = bf16_rne(r - bf16_bits_to_f32(m));
}
template <int D>
__device__ __forceinline__ void split_q(const f32x4* xa, const f32x4* xb, bool head_ok,
                                       QParts<D / 32>& q) {
    const float qscale = kLog2e / sqrtf((float)D);
#pragma unroll
    for (int ks = 0; ks < D / 32; ++ks) {
        const f32x4 x0 = xa[ks], x1 = xb[ks];
        u32x4 w3[3];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const float v0 = head_ok ? (e < 2 ? x0[2 * e] : x1[2 * e - 4]) * qscale : 0.f;
            const float v1 = head_ok ? (e < 2 ? x0[2 * e + 1] : x1[2 * e - 3]) * qscale : 0.f;
            uint16_t p0[3], p1[3];
            split3_bits(v0, p0[0], p0[1], p0[2]);
            split3_bits(v1, p1[0], p1[1], p1[2]);
#pragma unroll
            for (int i = 0; i < 3; ++i) w3[i][e] = (uint32_t)p0[i] | ((uint32_t)p1[i] << 16);
        }
#pragma unroll
        for (int i = 0; i < 3; ++i) q.part[i][ks] = as_bf16x8(w3[i]);
    }
}

// Writes the wave's (m, l, O^T) to LDS and combines the 4 waves.
template <int D>
__device__ __forceinline__ void finish_waves(const AttnParams& a, float (*sm_m)[16],
                                             float (*sm_l)[16], float (*sm_o)[16][D + 4],
                                             float m_run, float l_run, const f32x4* acc, int wv,
                                             int w, int c, int b, int g, int G, int part,
                                             int nparts) {
    const float l_tot = sum_over_rows(l_run);
    if (w == 0) {
        sm_m[wv][c] = m_run;
        sm_l[wv][c] = l_tot;
    }
    // lane (w, c) element v of tile md: O^T[16md + 4w + v][c]
#pragma unroll
    for (int md = 0; md < D / 16; ++md)
#pragma unroll
        for (int v = 0; v < 4; ++v) sm_o[wv][c][16 * md + 4 * w + v] = acc[md][v];
    __syncthreads();
    combine_waves<D>(a, sm_m, sm_l, sm_o, b, g, G, part, nparts);
}

template <int P, int D, bool kSparse>
__global__ __launch_bounds__(256) void attend_mfma_kernel(const AttnParams a) {
    static_assert(P == 64 && D % 32 == 0, "bf16 path: 64-token pages");
    constexpr int KS = D / 32;
    constexpr int MD = D / 16;
    __shared__ float sm_m[4][16], sm_l[4][16];
    __shared__ float sm_o[4][16][D + 4];

    const int lane = threadIdx.x & 63;
    const int wv = threadIdx.x >> 6;
    const int w = lane >> 4;
    const int c = lane & 15;
    const int S = a.num_splits;
    const int NPART = a.num_parts;
    const int item = blockIdx.x;
    const int part = item % NPART;
    const int g = (item / NPART) % a.num_kv_heads;
    const int b = item / (NPART * a.num_kv_heads);
    const int s = part * 4 + wv;  // this wave's split (may be past the last)
    const int Hkv = a.num_kv_heads;
    const int G = a.num_q_heads / Hkv;
    const bool head_ok = c < G;
    const int hq = g * G + (head_ok ? c : 0);

    const int seq_raw = a.seq_lens[b];
    const int summ_raw = a.summarized ? a.summarized[b] : 0;
    // sparse: this lane's list entry (slot s * pages_per_split + lane; a run
    // has at most 16 slots), read together with the sequence length; the
    // list is a readable device array even when k_sel = 0
    int j_list0 = 0;
    if constexpr (kSparse) {
        const int slot = s * a.pages_per_split + lane;
        j_list0 = a.sel_pages[((size_t)b * Hkv + g) * a.k_sel + (slot < a.k_sel ? slot : 0)];
        asm volatile("" ::"s"(seq_raw), "s"(summ_raw), "v"(j_list0));
    }
    const int seq = seq_raw < 0 ? 0 : seq_raw;
    int n_all = (seq + P - 1) / P;
    n_all = n_all > a.max_pages ? a.max_pages : n_all;
    // candidates (full pages with summaries); pages [cand, n_all) form the tail
    const int cand = candidate_pages(seq_raw, summ_raw, a.summarized != nullptr, P, a.max_pages);
    // dense: consecutive pages [first, first + count); sparse: slots
    // [first, first + count) of the selected list (pages_per_split per wave)
    SplitPages sp{0, 0};
    if (s < S) {
        if constexpr (kSparse) {
            const int slots = a.k_sel + 1;
            const int lo = s * a.pages_per_split;
            const int hi = lo + a.pages_per_split < slots ? lo + a.pages_per_split : slots;
            sp = {lo, hi > lo ? hi - lo : 0};
        } else {
            sp = split_pages(a, false, b, g, s, cand, n_all);
        }
    }

    QParts<KS> qp;
    float m_run = -INFINITY, l_run = 0.f;
    f32x4 acc[MD];
#pragma unroll
    for (int md = 0; md < MD; ++md) acc[md] = f32x4{0.f, 0.f, 0.f, 0.f};

    const uint16_t* kpool = static_cast<const uint16_t*>(a.k);
    const uint16_t* vpool = static_cast<const uint16_t*>(a.v);
    const int32_t* bt = a.block_table + (size_t)b * a.max_pages;

    // page descriptors: K and V of block ph (no records when absent)
    auto kpage = [&](int ph, bool present) {
        return page_rsrc(kpool + (present ? ((size_t)ph * Hkv + g) * P * D : 0), present,
                         2 * P * D);
    };
    auto vpage = [&](int ph, bool present) {
        return page_rsrc(vpool + (present ? ((size_t)ph * Hkv + g) * D * P : 0), present,
                         2 * P * D);
    };
    // Dense: page j of the run and its block; -1 / -1 when the block-table
    // entry is out of range.
    auto resolve = [&](int j, int& jl, int& pl) {
        const int ph = bt[j];
        const bool ok = ph >= 0 && ph < a.num_blocks;
        jl = ok ? j : -1;
        pl = ok ? ph : -1;
    };
    // Walks the valid pages (lanes of `todo`, lowest first) with one page
    // buffer: the next page's keys load while this page's values are used,
    // and its values while its own keys are.  Loads for a page past the end
    // are issued too (they fetch nothing): no load sits under a branch, so
    // each wait covers only the loads it needs.  `ready` runs once the
    // first page's loads are issued.
    auto walk = [&](uint64_t todo, int jl, int pl, auto&& ready) {
        auto take = [&](int& jj, int& ph) -> bool {
            const bool has = todo != 0;
            const int ln = has ? __builtin_ffsll((long long)todo) - 1 : 0;
            jj = __builtin_amdgcn_readlane(jl, ln);
            ph = __builtin_amdgcn_readlane(pl, ln);
            todo &= todo - 1;
            return has;
        };
        PageFrag<P, D> f;
        int j, ph;
        take(j, ph);
        load_page_k_rsrc<P, D>(kpage(ph, true), w, c, f);
        load_page_v_rsrc<P, D>(vpage(ph, true), w, c, f);
        ready();
        while (true) {
            const int nv = seq - j * P < P ? seq - j * P : P;  // valid tokens of the page
            int jn, pn;
            const bool more = take(jn, pn);
            f32x4 sc[PageFrag<P, D>::MT];
            page_scores<P, D>(f, nv, w, qp, sc);
            load_page_k_rsrc<P, D>(kpage(pn, more), w, c, f);
            page_values<P, D>(f, sc, nv, w, m_run, l_run, acc);
            load_page_v_rsrc<P, D>(vpage(pn, more), w, c, f);
            if (!more) break;
            j = jn;
        }
    };

    if constexpr (kSparse) {
        // A sparse run is one chunk (at most 16 slots).  Lane l's page is
        // slot sp.first + l, whose list entry was read up front; the slots
        // from k_sel on are the tail, pages cand, cand + 1, .. (normally just
        // the partial page), one per lane up to the wave's 64 lanes.  The
        // block-table read is unconditional (clamped to entry 0: the table
        // has at least one column) and goes out before the query's loads;
        // the page is checked once those are issued, and the query is split
        // only after the first page's loads are out.
        const int slot = sp.first + lane;
        const int tail = n_all - cand;  // pages without a summary
        // the wave whose slots include k_sel takes the tail (lanes from k_sel on)
        const bool tail_wave = s < S && sp.first <= a.k_sel && a.k_sel < sp.first + sp.count;
        int jc = -1;
        if (slot < a.k_sel)
            jc = (lane < sp.count && j_list0 >= 0 && j_list0 < cand) ? j_list0 : -1;
        else if (tail_wave && slot - a.k_sel < tail)
            jc = cand + (slot - a.k_sel);
        const int ph_raw = bt[jc >= 0 ? jc : 0];
        f32x4 xa[KS], xb[KS];
        load_q_raw<D>(a, b, hq, w, xa, xb);
        // keeps the query's loads ahead of the first use of ph_raw (which
        // waits for the block-table read)
        asm volatile("" ::: "memory");
        const bool ok = jc >= 0 && ph_raw >= 0 && ph_raw < a.num_blocks;
        const int jl = ok ? jc : -1, pl = ok ? ph_raw : -1;
        const uint64_t todo = __ballot(ok);
        bool split = false;
        if (todo != 0) walk(todo, jl, pl, [&] { split_q<D>(xa, xb, head_ok, qp); split = true; });
        // a tail longer than the lanes left for it: the rest, 64 pages a round
        const int in_wave = sp.first + kWave - a.k_sel;  // tail pages the first round took
        if (tail_wave) {
            for (int base = in_wave; base < tail; base += kWave) {
                const int t = base + lane;
                const int jt = t < tail ? cand + t : -1;
                const int pt = bt[jt >= 0 ? jt : 0];
                const bool okt = jt >= 0 && pt >= 0 && pt < a.num_blocks;
                const uint64_t todo2 = __ballot(okt);
                if (todo2 != 0)
                    walk(todo2, okt ? jt : -1, okt ? pt : -1, [&] {
                        if (!split) split_q<D>(xa, xb, head_ok, qp);
                        split = true;
                    });
            }
        }
    } else {
        {
            f32x4 xa[KS], xb[KS];
            load_q_raw<D>(a, b, hq, w, xa, xb);
            split_q<D>(xa, xb, head_ok, qp);
        }
        // The run's page indices and blocks are resolved up front, one lane
        // per page (64 at a time), so each page's K/V loads issue without
        // waiting for its block-table entry.
        for (int base = 0; base < sp.count; base += kWave) {
            const int n = sp.count - base < kWave ? sp.count - base : kWave;
            int jl = -1, pl = -1;
            if (lane < n) resolve(sp.first + base + lane, jl, pl);
            const uint64_t todo = __ballot(lane < n && jl >= 0);
            if (todo != 0) walk(todo, jl, pl, [] {});
        }
    }
    finish_waves<D>(a, sm_m, sm_l, sm_o, m_run, l_run, acc, wv, w, c, b, g, G, part, NPART);
}

// Sparse path (bf16, latency-bound at small batch): one workgroup per split
// (one selected page, or the partial last page), wave wv owns tokens
// [16wv, 16wv + 16), so each page is fetched by 4 waves at once.  Per wave:
//   S^T (16 tok x 16 h) = K_tile (16 x d) . q^T   v_mfma_f32_16x16x32_bf16, q in three parts
//   O^T (d x 16 h)     += V^T (d x 16 tok) . p^T  v_mfma_f32_16x16x16bf16_1k, p as hi + lo
// Lane (w, c) receives the scores of tokens 4w..4w+3 of its slice for head c,
// which are exactly its 4 contraction elements of the value product; its
// value operand is 4 consecutive tokens of one V^T row (8 bytes).
template <int P, int D>
__global__ __launch_bounds__(256) void attend_sparse_kernel(const AttnParams a) {
    static_assert(P == 64 && D % 32 == 0, "bf16 path: 64-token pages");
    constexpr int KS = D / 32;
    constexpr int MD = D / 16;
    __shared__ float sm_m[4][16], sm_l[4][16];
    __shared__ float sm_o[4][16][D + 4];

    const int lane = threadIdx.x & 63;
    const int wv = threadIdx.x >> 6;
    const int w = lane >> 4;
    const int c = lane & 15;
    const int S = a.num_splits;
    const int item = blockIdx.x;
    const int s = item % S;
    const int g = (item / S) % a.num_kv_heads;
    const int b = item / (S * a.num_kv_heads);
    const int Hkv = a.num_kv_heads;
    const int G = a.num_q_heads / Hkv;
    const bool head_ok = c < G;
    const int hq = g * G + (head_ok ? c : 0);
    const int tok0 = 16 * wv;
    // the query's loads go out first (they depend on nothing); it is split
    // once the page's loads are out, while they are in flight
    f32x4 xa[KS], xb[KS];
    load_q_raw<D>(a, b, hq, w, xa, xb);

    // The list entry of this split is read together with the sequence length
    // (it does not depend on it), and the block-table entry as soon as both
    // are in: three dependent reads become two.
    // (sel_pages is always a readable device array: with k_sel = 0 it is a
    // marker that is read but never used)
    const int seq_raw = a.seq_lens[b];
    const int summ_raw = a.summarized ? a.summarized[b] : 0;
    const int j_list = a.sel_pages[((size_t)b * Hkv + g) * a.k_sel + (s < a.k_sel ? s : 0)];
    // the values are consumed here, so all reads issue before one wait
    // (otherwise the list read is sunk into the branch that uses it)
    asm volatile("" ::"s"(seq_raw), "s"(summ_raw), "s"(j_list));
    const int seq = seq_raw < 0 ? 0 : seq_raw;
    int n_all = (seq + P - 1) / P;
    n_all = n_all > a.max_pages ? a.max_pages : n_all;
    const int cand =
        candidate_pages(seq_raw, summ_raw, a.summarized != nullptr, P, a.max_pages);
    SplitPages sp{0, 0};
    if (s < a.k_sel) {
        if (j_list >= 0 && j_list < cand) sp = {j_list, 1};
    } else if (n_all > cand) {
        sp = {cand, n_all - cand};  // pages without a summary (normally the partial page)
    }

    QParts<KS> qp;
    float m_run = -INFINITY, l_run = 0.f;
    f32x4 acc[MD];
#pragma unroll
    for (int md = 0; md < MD; ++md) acc[md] = f32x4{0.f, 0.f, 0.f, 0.f};
    // one page (pi = 0: also the query's loads and split); the tail split
    // walks its pages one after the other with the running max rescaled
    for (int pi = 0; pi < (sp.count > 0 ? sp.count : 1); ++pi) {
    const int jpg = sp.first + pi;
    int phys = sp.count ? a.block_table[(size_t)b * a.max_pages + jpg] : -1;
    const bool page_ok = sp.count && phys >= 0 && phys < a.num_blocks;
    phys = page_ok ? phys : 0;

    // page slice: K rows tok0 + c (4 x 16 B), V^T rows 16md + c at tokens tok0 + 4w (MD x 8 B)
    u32x4 kraw[KS];
    u32x2 vraw[MD];
    {
        const uint16_t* kp = static_cast<const uint16_t*>(a.k) + ((size_t)phys * Hkv + g) * P * D +
                             (size_t)(tok0 + c) * D;
        const uint16_t* vp = static_cast<const uint16_t*>(a.v) + ((size_t)phys * Hkv + g) * D * P +
                             tok0 + 4 * w;
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) kraw[ks] = *reinterpret_cast<const u32x4*>(kp + 32 * ks + 8 * w);
#pragma unroll
        for (int md = 0; md < MD; ++md)
            vraw[md] = *reinterpret_cast<const u32x2*>(vp + (size_t)(16 * md + c) * P);
    }

    if (pi == 0) split_q<D>(xa, xb, head_ok, qp);

    if (page_ok) {
        const int nv = seq - jpg * P < P ? seq - jpg * P : P;
        f32x4 sc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
            const bf16x8 kf = as_bf16x8(kraw[ks]);
            sc = mfma_16x16x32_bf16(kf, qp.part[2][ks], sc);
            sc = mfma_16x16x32_bf16(kf, qp.part[1][ks], sc);
            sc = mfma_16x16x32_bf16(kf, qp.part[0][ks], sc);
        }
        if (nv < P) {
#pragma unroll
            for (int v = 0; v < 4; ++v) sc[v] = tok0 + 4 * w + v < nv ? sc[v] : -INFINITY;
        }
        const float mx_page = max_over_rows(fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3])));
        const float mx = fmaxf(m_run, mx_page);
        if (mx != -INFINITY) {
            // earlier pages of the tail: rescale to the new running max
            if (m_run != -INFINITY && m_run != mx) {
                const float al = fast_exp2(m_run - mx);
                l_run *= al;
#pragma unroll
                for (int md = 0; md < MD; ++md) acc[md] *= al;
            }
            uint32_t ph[2], pl[2];
            float psum = 0.f;
#pragma unroll
            for (int e2 = 0; e2 < 2; ++e2) {
                const float p0 = fast_exp2(sc[2 * e2] - mx);
                const float p1 = fast_exp2(sc[2 * e2 + 1] - mx);
                psum += p0 + p1;
                uint16_t h0, l0, h1, l1;
                split_bf16(p0, h0, l0);
                split_bf16(p1, h1, l1);
                ph[e2] = (uint32_t)h0 | ((uint32_t)h1 << 16);
                pl[e2] = (uint32_t)l0 | ((uint32_t)l1 << 16);
            }
            m_run = mx;
            l_run += psum;
            const bf16x4 bhi = as_bf16x4(u32x2{ph[0], ph[1]});
            const bf16x4 blo = as_bf16x4(u32x2{pl[0], pl[1]});
#pragma unroll
            for (int md = 0; md < MD; ++md) {
                u32x2 vr = vraw[md];
                if (nv < P) {  // absent tokens: p is 0, their bits may be NaN
#pragma unroll
                    for (int e2 = 0; e2 < 2; ++e2) {
                        const int tk = tok0 + 4 * w + 2 * e2;
                        vr[e2] &= (tk < nv ? 0x0000ffffu : 0u) | (tk + 1 < nv ? 0xffff0000u : 0u);
                    }
                }
                const bf16x4 vf = as_bf16x4(vr);
                acc[md] = mfma_16x16x16_bf16(vf, bhi, acc[md]);
                acc[md] = mfma_16x16x16_bf16(vf, blo, acc[md]);
            }
        }
    }
    }  // pages of the split
    const float l_tot = sum_over_rows(l_run);
    if (w == 0) {
        sm_m[wv][c] = m_run;
        sm_l[wv][c] = l_tot;
    }
#pragma unroll
    for (int md = 0; md < MD; ++md)
#pragma unroll
        for (int v = 0; v < 4; ++v) sm_o[wv][c][16 * md + 4 * w + v] = acc[md][v];
    __syncthreads();
    combine_waves<D>(a, sm_m, sm_l, sm_o, b, g, G, s, S);
}

// fp32 caches: plain VALU loops, one workgroup per split (small shapes).
template <int P, int D, bool kSparse>
__global__ __launch_bounds__(256) void attend_f32_kernel(const AttnParams a) {
    __shared__ float qs[16][D];
    __shared__ float sc[16][P];
    __shared__ float os[16][D];
    __shared__ float mrun[16], lrun[16], alpha[16];

    const int S = a.num_splits;
    const int item = blockIdx.x;
    const int s = item % S;
    const int g = (item / S) % a.num_kv_heads;
    const int b = item / (S * a.num_kv_heads);
    const int Hkv = a.num_kv_heads;
    const int G = a.num_q_heads / Hkv;
    const int t = threadIdx.x;
    const int seq = a.seq_lens[b] < 0 ? 0 : a.seq_lens[b];
    int n_all = (seq + P - 1) / P;
    n_all = n_all > a.max_pages ? a.max_pages : n_all;
    const int cand = attn_candidates(a, b, seq);
    const SplitPages sp = split_pages(a, kSparse, b, g, s, cand, n_all);

    const float qscale = kLog2e / sqrtf((float)D);
    for (int i = t; i < G * D; i += 256) {
        const int h = i / D, d = i % D;
        qs[h][d] = a.q[((size_t)b * a.num_q_heads + g * G + h) * D + d] * qscale;
        os[h][d] = 0.f;
    }
    if (t < G) {
        mrun[t] = -INFINITY;
        lrun[t] = 0.f;
    }
    __syncthreads();

    const float* kpool = static_cast<const float*>(a.k);
    const float* vpool = static_cast<const float*>(a.v);
    for (int pi = 0; pi < sp.count; ++pi) {
        const int j = sp.first + pi;
        const int phys = a.block_table[(size_t)b * a.max_pages + j];
        if (phys < 0 || phys >= a.num_blocks) continue;  // uniform
        const int nv = seq - j * P < P ? seq - j * P : P;
        const float* kp = kpool + ((size_t)phys * Hkv + g) * P * D;
        const float* vp = vpool + ((size_t)phys * Hkv + g) * D * P;
        for (int i = t; i < G * P; i += 256) {
            const int h = i / P, tok = i % P;
            float x = -INFINITY;
            if (tok < nv) {
                x = 0.f;
                for (int d = 0; d < D; ++d) x += qs[h][d] * kp[(size_t)tok * D + d];
            }
            sc[h][tok] = x;
        }
        __syncthreads();
        if (t < G) {
            float mx = -INFINITY;
            for (int tok = 0; tok < nv; ++tok) mx = fmaxf(mx, sc[t][tok]);
            const float m_new = fmaxf(mrun[t], mx);
            const float al = m_new == -INFINITY ? 1.f : fast_exp2(mrun[t] - m_new);
            float sum = 0.f;
            for (int tok = 0; tok < P; ++tok) {
                const float p = tok < nv && m_new != -INFINITY ? fast_exp2(sc[t][tok] - m_new) : 0.f;
                sc[t][tok] = p;
                sum += p;
            }
            lrun[t] = lrun[t] * al + sum;
            mrun[t] = m_new;
            alpha[t] = al;
        }
        __syncthreads();
        for (int i = t; i < G * D; i += 256) {
            const int h = i / D, d = i % D;
            float o = os[h][d] * alpha[h];
            for (int tok = 0; tok < nv; ++tok) o += sc[h][tok] * vp[(size_t)d * P + tok];
            os[h][d] = o;
        }
        __syncthreads();
    }
    for (int i = t; i < G * D; i += 256) {
        const int h = i / D, d = i % D;
        const size_t row = ((size_t)b * a.num_q_heads + g * G + h) * a.num_parts + s;
        a.part_o[row * D + d] = os[h][d];
        if (d == 0) {
            a.part_ml[2 * row] = mrun[h];
            a.part_ml[2 * row + 1] = lrun[h];
        }
    }
}

// DPP row rotation by 8 lanes (within each 16-lane row): lane l reads l ^ 8.
constexpr int kDppRowRor8 = 0x128;

// A running softmax state: max, sum and unnormalised output (4 dims).
struct MergeState {
    float m, l;
    f32x4 o;
};
// The merge of two states, the same bits whichever argument comes first
// (products formed separately, then added; no fused multiply-add), so the
// two lanes of an exchanged pair end up holding one state.  An empty state
// (m = -inf, l = 0) contributes nothing.
__device__ __forceinline__ MergeState merge_states(const MergeState& x, const MergeState& y) {
#pragma clang fp contract(off)
    const float M = fmaxf(x.m, y.m);
    const float wx = x.m == -INFINITY ? 0.f : fast_exp2(x.m - M);
    const float wy = y.m == -INFINITY ? 0.f : fast_exp2(y.m - M);
    MergeState r;
    r.m = M;
    r.l = x.l * wx + y.l * wy;
#pragma unroll
    for (int e = 0; e < 4; ++e) r.o[e] = x.o[e] * wx + y.o[e] * wy;
    return r;
}
// Lane l and lane l ^ 8 (DPP row rotation by 8 within each 16-lane row).
__device__ __forceinline__ MergeState merge_xor8(const MergeState& x) {
    MergeState y;
    y.m = dpp<kDppRowRor8>(x.m);
    y.l = dpp<kDppRowRor8>(x.l);
#pragma unroll
    for (int e = 0; e < 4; ++e) y.o[e] = dpp<kDppRowRor8>(x.o[e]);
    return merge_states(x, y);
}
// Lane l with lane l ^ 16 (kRow16) or l ^ 32: the gfx950 row swaps of a
// register with itself give each lane the pair (own, partner) in some order,
// which the symmetric merge does not need to know.
template <bool kRow16>
__device__ __forceinline__ MergeState merge_swap(const MergeState& x) {
    auto sw = [](float v) {
        const auto p = kRow16 ? __builtin_amdgcn_permlane16_swap(__float_as_uint(v),
                                                                 __float_as_uint(v), false, false)
                              : __builtin_amdgcn_permlane32_swap(__float_as_uint(v),
                                                                 __float_as_uint(v), false, false);
        return f32x2{__uint_as_float(p[0]), __uint_as_float(p[1])};
    };
    MergeState u, v;
    const f32x2 mm = sw(x.m), ll = sw(x.l);
    u.m = mm[0];
    v.m = mm[1];
    u.l = ll[0];
    v.l = ll[1];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const f32x2 oo = sw(x.o[e]);
        u.o[e] = oo[0];
        v.o[e] = oo[1];
    }
    return merge_states(u, v);
}

// Merge of the partials of one (b, h).  Grid: (b, h) x 32-dim chunk;
// thread t handles dims [32*chunk + 4*(t%8), +4) over the partials
// p = t/8, t/8 + 32, ... with a running (max, sum, output) rescaled as each
// partial arrives (one round of loads, no max pre-pass).  The 32 running
// states of each 4 dims are then merged as a tree: the 8 of a wave by lane
// exchanges (lanes l ^ 8, l ^ 16, l ^ 32), the 4 waves' results in order
// through LDS.  Deterministic: the merge order depends only on the shapes.
template <int D>
__global__ __launch_bounds__(256) void merge_kernel(const AttnParams a) {
    __shared__ f32x4 so[4][8];
    __shared__ float sm[4][8], sl[4][8];
    const int bh = blockIdx.x;
    const int chunk = blockIdx.y;
    const int t = threadIdx.x;
    const int NP = a.num_parts;
    const float* ml = a.part_ml + (size_t)bh * NP * 2;
    const float* po = a.part_o + (size_t)bh * NP * D + 32 * chunk;

    const int d4 = t & 7, part = t >> 3;
    float m_run = -INFINITY, l_run = 0.f;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    // Branch-free so that every partial's loads are issued before any is
    // used; an empty partial (l = 0) leaves the running state unchanged.
#pragma unroll 4
    for (int s = part; s < NP; s += 32) {
        const f32x2 m_l = *reinterpret_cast<const f32x2*>(ml + 2 * s);
        const f32x4 o = *reinterpret_cast<const f32x4*>(po + (size_t)s * D + 4 * d4);
        const bool ok = m_l[1] > 0.f;
        const float mn = fmaxf(m_run, m_l[0]);
        const float w_old = fast_exp2(m_run - mn);  // 0 while nothing is held
        const float w_new = fast_exp2(m_l[0] - mn);
        const f32x4 acc_n = acc * w_old + o * w_new;
        const float l_n = l_run * w_old + m_l[1] * w_new;
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[e] = ok ? acc_n[e] : acc[e];
        l_run = ok ? l_n : l_run;
        m_run = ok ? mn : m_run;
    }
    // -inf with l = 0 when the thread held nothing
    MergeState st{m_run, l_run, acc};
    st = merge_xor8(st);
    st = merge_swap<true>(st);
    st = merge_swap<false>(st);
    const int wv = t >> 6;
    if ((t & 63) < 8) {
        so[wv][d4] = st.o;
        sm[wv][d4] = st.m;
        sl[wv][d4] = st.l;
    }
    __syncthreads();
    if (t < 8) {
        MergeState f{sm[0][t], sl[0][t], so[0][t]};
#pragma unroll
        for (int w = 1; w < 4; ++w) f = merge_states(f, MergeState{sm[w][t], sl[w][t], so[w][t]});
        const float M = f.m, L = f.l;
        const f32x4 o = f.o;
        const size_t base = (size_t)bh * D + 32 * chunk + 4 * t;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const float res = L > 0.f ? o[e] / L : 0.f;
            if (a.bf16)
                static_cast<uint16_t*>(a.out)[base + e] = f32_to_bf16_bits(res);
            else
                static_cast<float*>(a.out)[base + e] = res;
        }
        if (chunk == 0 && t == 0 && a.out_lse)
            a.out_lse[bh] = L > 0.f ? (M + fast_log2(L)) * kLn2 : -INFINITY;
    }
}

// Sparse lists with at least this many (b, g, slot) pages run on the
// wave-per-page kernel (bandwidth-bound batches); fewer run one workgroup
// per page (latency-bound single sequences).
constexpr long kSparseWavePages = 1024;

template <int P, int D>
hipError_t launch_pd(AttnParams p, hipStream_t s) {
    const bool sparse = p.sel_pages != nullptr;
    if (p.bf16) {
        if constexpr (P == 64) {
            const long slots = (long)p.k_sel + 1;
            const long total = (long)p.batch * p.num_kv_heads * slots;
            if (sparse && total < kSparseWavePages) {  // few pages: one workgroup per page
                p.num_parts = p.num_splits;
                const unsigned blocks = (unsigned)((long)p.batch * p.num_kv_heads * p.num_splits);
                if (blocks > 0)
                    hipLaunchKernelGGL((attend_sparse_kernel<P, D>), dim3(blocks), dim3(256), 0, s,
                                       p);
            } else if (sparse) {  // many pages: one wave per run of selected pages
                // ~1024 waves (one per SIMD), each walking its run of pages: measured
                // faster than more, shorter runs, also with two waves resident per
                // SIMD (256 registers, a few spills)
                long pps = (total + 1023) / 1024;
                pps = pps < 1 ? 1 : (pps > 16 ? 16 : pps);
                p.pages_per_split = (int)pps;
                p.num_splits = (int)((slots + pps - 1) / pps);
                p.num_parts = (p.num_splits + 3) / 4;
                const unsigned blocks = (unsigned)((long)p.batch * p.num_kv_heads * p.num_parts);
                if (blocks > 0)
                    hipLaunchKernelGGL((attend_mfma_kernel<P, D, true>), dim3(blocks), dim3(256),
                                       0, s, p);
            } else {  // one wave per run of pages, 4 runs per workgroup
                p.num_parts = (p.num_splits + 3) / 4;
                const unsigned blocks = (unsigned)((long)p.batch * p.num_kv_heads * p.num_parts);
                if (blocks > 0)
                    hipLaunchKernelGGL((attend_mfma_kernel<P, D, false>), dim3(blocks), dim3(256),
                                       0, s, p);
            }
        } else {
            return hipErrorInvalidValue;
        }
    } else {
        p.num_parts = p.num_splits;
        const unsigned blocks = (unsigned)((long)p.batch * p.num_kv_heads * p.num_splits);
        if (blocks > 0) {
            if (sparse)
                hipLaunchKernelGGL((attend_f32_kernel<P, D, true>), dim3(blocks), dim3(256), 0, s,
                                   p);
            else
                hipLaunchKernelGGL((attend_f32_kernel<P, D, false>), dim3(blocks), dim3(256), 0, s,
                                   p);
        }
    }
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const unsigned rows = (unsigned)(p.batch * p.num_q_heads);
    if (rows == 0) return hipSuccess;
    hipLaunchKernelGGL((merge_kernel<D>), dim3(rows, D / 32), dim3(256), 0, s, p);
    return hipGetLastError();
}

}  // namespace

bool attend_supported(int bf16, int page_size, int head_dim) {
    if (head_dim != 64 && head_dim != 128) return false;
    if (bf16) return page_size == 64;
    return page_size == 16 || page_size == 64;
}

int dense_pages_per_split(int batch, int num_kv_heads, int max_pages) {
    // one wave per split; aim for ~2048 waves (8 per CU, the occupancy of the
    // dense kernel) so that one round covers the cache
    long pps = (long)batch * num_kv_heads * max_pages / 2048;
    if (pps < 1) pps = 1;
    if (pps > 256) pps = 256;
    return (int)pps;
}

hipError_t launch_attend(const AttnParams& p, hipStream_t s) {
    if (p.page_size == 16 && p.head_dim == 64) return launch_pd<16, 64>(p, s);
    if (p.page_size == 16 && p.head_dim == 128) return launch_pd<16, 128>(p, s);
    if (p.page_size == 64 && p.head_dim == 64) return launch_pd<64, 64>(p, s);
    return launch_pd<64, 128>(p, s);
}

}  // namespace locks
