// Top-k page selection per (sequence, KV group): the k pages with the
// largest estimated log-mass (gist.science technical summary, section 2,
// Reconstructie en Selectie: pages are ranked by estimated mass), equal
// fp32 values broken toward the lower page index, written in ascending page
// order.
//
// One 1024-thread workgroup per (b, g).  Masses become order-preserving
// 32-bit keys.  The selection is defined on the 64-bit key
// (key << 32 | ~page), a total order, so the result is unique and
// deterministic.
//
// Fast path (k <= 64):
//  1. Bound.  Every thread reduces its share of the keys to a maximum;
//     64 groups of 16 threads, each group taking every 64th thread (so every
//     group is populated once 64 threads hold keys), report their largest.
//     The k-th largest group maximum T is a real key with at least k keys
//     >= T, so every winner is >= T: a lower bound that usually admits only
//     a few dozen candidates.  T is found by ranking the 64 group maxima,
//     16 threads per value and a DPP row sum.
//     With the scan's run maxima (maxima of runs of 16 consecutive pages,
//     each a real key) the threads hold run maxima instead of masses, dealt
//     so that each group is one row of 16 threads (its maximum a DPP row
//     reduction, no LDS round), and only the runs whose maximum reaches T
//     are then read, one page per thread (more than 256 such runs: the
//     masses are read instead).
//  2. Keys >= T are appended to an LDS list (wave ballot + one LDS atomic per
//     wave; order irrelevant).  Each candidate's rank is counted against the
//     whole list by 16 threads and a row sum; rank < k wins.
//  3. A winner's output slot is the number of winners with a lower page,
//     counted the same way; its mass is recovered from the key.
// Fallback (k > 64 or more than 1024 candidates): bitwise radix select of the
// k-th largest key (one bit per step, counts from wave ballots), then two
// block prefix sums in page order take the keys above it and the
// lowest-page ties.
#include "device_common.hpp"
#include "launchers.hpp"

namespace locks {

namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / kWave;
constexpr int kMaxPer = kTopkMaxPages / kThreads;  // keys per thread
constexpr int kVecPer = kMaxPer / 4;               // 16-byte loads per thread
constexpr int kFastK = 64;
constexpr int kCandCap = 1024;
constexpr int kMaxRuns = kTopkMaxPages / kRunPages;  // 2048
constexpr int kRunPer = kMaxRuns / kThreads;         // run maxima per thread
constexpr int kListPer = 4;                          // pages of listed runs per thread
constexpr int kListCap = kListPer * kThreads / kRunPages;  // runs read (256)

__device__ __forceinline__ uint32_t popc64(unsigned long long m) { return __popcll(m); }

// Inverse of orderable_bits (up to the sign of zero).
__device__ __forceinline__ float key_to_float(uint32_t k) {
    return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

__device__ __forceinline__ uint32_t lanes_below(unsigned long long m) {
    return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

// Appends `item` for the lanes with `hit` to list[] at *count (one LDS atomic
// per wave); entries past `cap` are dropped but still counted.
template <typename T>
__device__ __forceinline__ void wave_append(bool hit, T item, T* list, uint32_t* count, int cap) {
    const unsigned long long m = __ballot(hit);
    if (m) {
        uint32_t base = 0;
        if ((threadIdx.x & 63) == 0) base = atomicAdd(count, (uint32_t)popc64(m));
        base = __builtin_amdgcn_readfirstlane(base);
        const uint32_t slot = base + lanes_below(m);
        if (hit && slot < (uint32_t)cap) list[slot] = item;
    }
}

// The k-th largest of 64 group maxima of the threads' maxima.  kRows: group
// i is the 16 threads of row i (t / 16 = i), whose maxima meet in DPP, and
// the caller deals its items so that a row holds what a strided group would;
// otherwise group i = threads i, i+64, ..., i+960, gathered through LDS.
// Contains one (kRows) or two more barriers; every thread gets T.
template <bool kRows>
__device__ __forceinline__ uint32_t group_bound(uint32_t my_max, int k, uint32_t* s_tmax,
                                                uint32_t* s_gmax, uint32_t* s_T) {
    const int t = threadIdx.x, i_row = t >> 4, q = t & 15;
    uint32_t x = my_max;
    if constexpr (!kRows) {
        s_tmax[t] = my_max;
        __syncthreads();
        x = s_tmax[i_row + 64 * q];
    }
    const uint32_t gm = umax_in_row(x);
    if (q == 0) s_gmax[i_row] = gm;
    __syncthreads();
    // rank of group maximum i_row (larger first, then lower index): the ranks
    // are a permutation of 0..63, so exactly one group has rank k-1
    const uint32_t v = s_gmax[i_row];
    int cnt = 0;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const int u = 4 * q + e;
        const uint32_t o = s_gmax[u];
        cnt += (o > v || (o == v && u < i_row)) ? 1 : 0;
    }
    const int rank = (int)sum_in_row((float)cnt);
    if (q == 0 && rank == k - 1) *s_T = v;
    __syncthreads();
    return *s_T;
}

// For larger k: the k-th largest of the 128 values formed by the two
// largest thread maxima of each of the 64 groups.  The two come from
// different threads, so they are keys of different pages, and at least k
// keys are >= the result: a lower bound on the k-th largest key, tighter
// than group_bound's once k approaches 64.  Key 0 marks an absent value.
// Groups as in group_bound.  Every thread gets T.  s_gmax holds 128 entries.
template <bool kRows>
__device__ __forceinline__ uint32_t group_bound2(uint32_t my_max, int k, uint32_t* s_tmax,
                                                 uint32_t* s_gmax, uint32_t* s_T) {
    const int t = threadIdx.x, i_row = t >> 4, q = t & 15;
    uint32_t x = my_max;
    if constexpr (!kRows) {
        s_tmax[t] = my_max;
        __syncthreads();
        x = s_tmax[i_row + 64 * q];
    }
    const uint32_t m1 = umax_in_row(x);
    // the second largest: the row's maximum without its first holder
    const unsigned long long eq = __ballot(x == m1);
    const uint32_t row_eq = (uint32_t)(eq >> (16 * ((t & 63) >> 4))) & 0xffffu;
    const int first = __builtin_ctz(row_eq);  // the row's own lane holds m1
    const uint32_t m2 = umax_in_row(q == first ? 0u : x);
    if (q == 0) {
        s_gmax[i_row] = m1;
        s_gmax[64 + i_row] = m2;
    }
    __syncthreads();
    // ranks of values i_row and 64 + i_row (larger first, then lower index):
    // a permutation of 0..127, so exactly one value has rank k-1
    const uint32_t v1 = s_gmax[i_row], v2 = s_gmax[64 + i_row];
    int c1 = 0, c2 = 0;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const int u = 8 * q + e;
        const uint32_t o = s_gmax[u];
        c1 += (o > v1 || (o == v1 && u < i_row)) ? 1 : 0;
        c2 += (o > v2 || (o == v2 && u < 64 + i_row)) ? 1 : 0;
    }
    const int r1 = (int)sum_in_row((float)c1), r2 = (int)sum_in_row((float)c2);
    if (q == 0 && r1 == k - 1) *s_T = v1;
    if (q == 0 && r2 == k - 1) *s_T = v2;
    __syncthreads();
    return *s_T;
}

// Ranks the C (<= 1024) candidates of s_cand and writes the k (<= 64)
// winners in ascending page order.  Candidate i is handled by the 16
// threads of row i % 64 (rows loop over blocks of 64 candidates), each
// comparing it with every 16th block of 4 candidates; the row sum is its
// rank.  Contains one barrier.
__device__ __forceinline__ void rank_and_emit(const unsigned long long* s_cand, int C, int k,
                                              uint32_t* s_win, int32_t* out_sel, float* out_mass) {
    const int t = threadIdx.x, i_row = t >> 4, q = t & 15;
    for (int i0 = 0; i0 < C; i0 += 64) {  // uniform
        const int i = i0 + i_row;
        const unsigned long long mine = i < C ? s_cand[i] : 0ull;
        int cnt = 0;
        for (int u0 = 0; u0 < C; u0 += 64) {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int u = u0 + 4 * q + e;
                cnt += (u < C && s_cand[u < C ? u : 0] > mine) ? 1 : 0;
            }
        }
        const int rank = (int)sum_in_row((float)cnt);
        if (q == 0 && i < C && rank < k) s_win[rank] = (uint32_t)i;  // winner of rank r
    }
    __syncthreads();
    // output slot of winner i_row = winners with a lower page
    if (i_row < k) {
        const unsigned long long mine = s_cand[s_win[i_row]];
        const uint32_t my_page = 0xffffffffu - (uint32_t)mine;
        int cnt = 0;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int u = 4 * q + e;
            const uint32_t pu = 0xffffffffu - (uint32_t)s_cand[s_win[u < k ? u : 0]];
            cnt += (u < k && pu < my_page) ? 1 : 0;
        }
        const int pos = (int)sum_in_row((float)cnt);
        if (q == 0) {
            out_sel[pos] = (int32_t)my_page;
            if (out_mass) out_mass[pos] = key_to_float((uint32_t)(mine >> 32));
        }
    }
}

// Exclusive prefix sum over the workgroup (thread order); buf holds kWaves
// entries and must not be reused until every thread has passed the next
// barrier.
__device__ __forceinline__ uint32_t block_exclusive_scan(uint32_t v, uint32_t* buf,
                                                         uint32_t& total) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    uint32_t x = v;
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
        const uint32_t y = __shfl_up(x, off, kWave);
        if (lane >= off) x += y;
    }
    if (lane == kWave - 1) buf[wave] = x;
    __syncthreads();
    uint32_t before = 0, tot = 0;
#pragma unroll
    for (int w2 = 0; w2 < kWaves; ++w2) {
        const uint32_t s = buf[w2];
        before += w2 < wave ? s : 0u;
        tot += s;
    }
    total = tot;
    return before + x - v;
}

__global__ __launch_bounds__(kThreads) void topk_kernel(const TopkParams a) {
    __shared__ uint32_t s_tmax[kThreads];
    __shared__ uint32_t s_gmax[128];
    __shared__ uint32_t s_T;
    __shared__ uint32_t s_count[2];  // runs listed, candidates
    __shared__ uint32_t s_list[kListCap];
    __shared__ uint32_t s_win[kFastK];
    __shared__ unsigned long long s_cand[kCandCap];
    __shared__ uint32_t cnt[3][kWaves];
    __shared__ uint32_t scan_a[kWaves], scan_b[kWaves];

    const int bg = blockIdx.x;
    const int b = bg / a.num_kv_heads;
    const int t = threadIdx.x;
    const int wave = t >> 6;
    const int lane = t & 63;

    // The run maxima this thread may need (runs 1024 i + run_of_thread, i =
    // 0, 1) are read together with the sequence length, clamped to the
    // table's runs; which of them hold full pages is decided once the length
    // is in.  Runs are dealt so that row i of 16 threads holds runs i, i + 64,
    // ..., i + 960 (and 1024 + those): the 64 strided groups of the bound,
    // each in one DPP row, with every group populated once 64 runs exist.
    const int run_of_thread = 64 * (t & 15) + (t >> 4);
    const int nruns_all = (a.max_pages + kRunPages - 1) / kRunPages;
    const int seq_raw = a.seq_lens[b];
    const int summ_raw = a.summarized ? a.summarized[b] : 0;
    float rmv[kRunPer];
#pragma unroll
    for (int i = 0; i < kRunPer; ++i) rmv[i] = 0.f;
    if (a.run_max) {
        const float* rm = a.run_max + (size_t)bg * nruns_all;
#pragma unroll
        for (int i = 0; i < kRunPer; ++i) {
            const int r = i * kThreads + run_of_thread;
            rmv[i] = rm[r < nruns_all ? r : nruns_all - 1];
        }
    }
    // both reads issue before one wait (the run-maxima reads would otherwise
    // be sunk below the branches on the length)
    asm volatile("" ::"s"(seq_raw), "s"(summ_raw), "v"(rmv[0]), "v"(rmv[kRunPer - 1]));
    // candidates: the full pages whose summaries exist
    const int n =
        candidate_pages(seq_raw, summ_raw, a.summarized != nullptr, a.page_size, a.max_pages);
    const int k = a.k_req < n ? a.k_req : n;
    const float* row = a.page_logmass + (size_t)bg * a.max_pages;
    int32_t* out_sel = a.sel_pages + (size_t)bg * a.width;
    float* out_mass = a.sel_logmass ? a.sel_logmass + (size_t)bg * a.width : nullptr;

    for (int s = k + t; s < a.width; s += kThreads) {  // unused slots
        out_sel[s] = -1;
        if (out_mass) out_mass[s] = -INFINITY;
    }
    if (k <= 0) return;  // uniform over the workgroup
    if (k == n) {        // every full page wins, already in page order
        for (int j = t; j < n; j += kThreads) {
            out_sel[j] = j;
            if (out_mass) out_mass[j] = row[j];
        }
        return;
    }

    uint32_t key[kMaxPer];
    if (k <= kFastK) {
        if (t == 0) {
            s_count[0] = 0;
            s_count[1] = 0;
        }
        bool done = false;
        if (a.run_max) {
            // ---- bound from the run maxima (dealt as above)
            const int nruns = (n + kRunPages - 1) / kRunPages;  // runs holding full pages
            uint32_t rkey[kRunPer];
            uint32_t my_max = 0;
#pragma unroll
            for (int i = 0; i < kRunPer; ++i) {
                const int r = i * kThreads + run_of_thread;
                rkey[i] = r < nruns ? orderable_bits(rmv[i]) : 0u;
                my_max = rkey[i] > my_max ? rkey[i] : my_max;
            }
            const uint32_t T = k > 32 ? group_bound2<true>(my_max, k, s_tmax, s_gmax, &s_T)
                                      : group_bound<true>(my_max, k, s_tmax, s_gmax, &s_T);
#pragma unroll
            for (int i = 0; i < kRunPer; ++i)
                wave_append<uint32_t>(rkey[i] != 0u && rkey[i] >= T,
                                      (uint32_t)(i * kThreads + run_of_thread), s_list,
                                      &s_count[0], kListCap);
            __syncthreads();
            const int nlist = (int)s_count[0];
            if (nlist <= kListCap) {
                // page t%16 of listed runs t/16 + 64 m (m < kListPer) per thread, all
                // loads in flight together; candidates are the keys >= T (more than
                // kCandCap of them fall back to the exact search below)
                const int i_row = t >> 4;
                float mv[kListPer];
#pragma unroll
                for (int m = 0; m < kListPer; ++m) {
                    const int li = i_row + 64 * m;
                    const int j = li < nlist ? (int)s_list[li] * kRunPages + (t & 15) : 0;
                    mv[m] = row[j < n ? j : 0];
                }
#pragma unroll
                for (int m = 0; m < kListPer; ++m) {
                    const int li = i_row + 64 * m;
                    const int j = li < nlist ? (int)s_list[li] * kRunPages + (t & 15) : n;
                    const uint32_t kk = orderable_bits(mv[m]);
                    const bool hit = j < n && kk >= T;
                    const unsigned long long ck = ((unsigned long long)kk << 32) |
                                                  (unsigned long long)(0xffffffffu - (uint32_t)j);
                    wave_append<unsigned long long>(hit, ck, s_cand, &s_count[1], kCandCap);
                }
                __syncthreads();
                done = true;
            } else if (t == 0) {
                s_count[1] = 0;  // read every mass below
            }
        }
        if (!done) {
            // ---- bound from the masses themselves.  Aligned rows: key slot
            // 4i + e of thread t is page 4(1024 i + t) + e; otherwise page
            // 1024 s + t.  Loads are unconditional (clamped to a vector / page
            // that exists) so they are all in flight together; key 0 marks
            // "absent".
            const bool vec =
                (reinterpret_cast<uintptr_t>(row) & 15u) == 0 && (a.max_pages & 3) == 0;
            uint32_t my_max = 0;
            if (vec) {
                const int nv = (n + 3) >> 2;
                const f32x4* row4 = reinterpret_cast<const f32x4*>(row);
#pragma unroll
                for (int i = 0; i < kVecPer; ++i) {
                    const int v = i * kThreads + t;
                    const f32x4 x = row4[v < nv ? v : nv - 1];
#pragma unroll
                    for (int e = 0; e < 4; ++e) {
                        const bool ok = v < nv && 4 * v + e < n;
                        key[4 * i + e] = ok ? orderable_bits(x[e]) : 0u;
                        my_max = key[4 * i + e] > my_max ? key[4 * i + e] : my_max;
                    }
                }
            } else {
#pragma unroll
                for (int s = 0; s < kMaxPer; ++s) {
                    const int j = s * kThreads + t;
                    const float v = row[j < n ? j : n - 1];
                    key[s] = j < n ? orderable_bits(v) : 0u;
                    my_max = key[s] > my_max ? key[s] : my_max;
                }
            }
            const uint32_t T = group_bound<false>(my_max, k, s_tmax, s_gmax, &s_T);
#pragma unroll
            for (int s = 0; s < kMaxPer; ++s) {
                const int j = vec ? 4 * ((s >> 2) * kThreads + t) + (s & 3) : s * kThreads + t;
                wave_append<unsigned long long>(
                    key[s] != 0u && key[s] >= T,
                    ((unsigned long long)key[s] << 32) |
                        (unsigned long long)(0xffffffffu - (uint32_t)j),
                    s_cand, &s_count[1], kCandCap);
            }
            __syncthreads();
        }
        const int C = (int)s_count[1];  // >= k
        if (C <= kCandCap) {
            rank_and_emit(s_cand, C, k, s_win, out_sel, out_mass);
            return;
        }
        __syncthreads();  // the candidate list is abandoned: too many ties at the bound
    }

    // ---- fallback: exact bitwise search for the k-th largest key, on the
    // contiguous chunk layout: thread t holds pages [t c, t c + c)
    const int c = (n + kThreads - 1) / kThreads;
    const int j0 = t * c;
#pragma unroll
    for (int i = 0; i < kMaxPer; ++i) {
        const int j = j0 + i;
        const float v = row[j < n ? j : n - 1];
        key[i] = (i < c && j < n) ? orderable_bits(v) : 0u;
    }
    uint32_t tau = 0;
    for (int bit = 31; bit >= 0; --bit) {
        const uint32_t cand_t = tau | (1u << bit);
        uint32_t cn = 0;
#pragma unroll
        for (int i = 0; i < kMaxPer; ++i) cn += (i < c && key[i] >= cand_t) ? 1u : 0u;
        // wave sum of the per-thread counts
#pragma unroll
        for (int m = 1; m < kWave; m <<= 1) cn += __shfl_xor(cn, m, kWave);
        if (lane == 0) cnt[bit & 1][wave] = cn;
        __syncthreads();
        uint32_t total = 0;
#pragma unroll
        for (int w2 = 0; w2 < kWaves; ++w2) total += cnt[bit & 1][w2];
        if (total >= (uint32_t)k) tau = cand_t;
    }
    uint32_t above = 0, eq_mine = 0, gt_mine = 0;
#pragma unroll
    for (int i = 0; i < kMaxPer; ++i) {
        if (i < c) {
            gt_mine += key[i] > tau ? 1u : 0u;
            eq_mine += key[i] == tau ? 1u : 0u;
        }
    }
    uint32_t eq_total = 0;
    const uint32_t eq_before = block_exclusive_scan(eq_mine, scan_a, eq_total);
    {
        uint32_t g = gt_mine;
#pragma unroll
        for (int m = 1; m < kWave; m <<= 1) g += __shfl_xor(g, m, kWave);
        if (lane == 0) cnt[2][wave] = g;
    }
    __syncthreads();
#pragma unroll
    for (int w2 = 0; w2 < kWaves; ++w2) above += cnt[2][w2];
    const uint32_t need = (uint32_t)k - above;  // ties at tau to take, lowest page first
    // winners of this thread's chunk, in page order
    uint32_t sel_mine = 0, eq_seen = eq_before;
#pragma unroll
    for (int i = 0; i < kMaxPer; ++i) {
        if (i < c) {
            const bool eq = key[i] == tau;
            if (key[i] > tau || (eq && eq_seen < need)) ++sel_mine;
            if (eq) ++eq_seen;
        }
    }
    uint32_t sel_total = 0;
    uint32_t pos = block_exclusive_scan(sel_mine, scan_b, sel_total);
    eq_seen = eq_before;
#pragma unroll
    for (int i = 0; i < kMaxPer; ++i) {
        if (i < c) {
            const bool eq = key[i] == tau;
            if (key[i] > tau || (eq && eq_seen < need)) {
                out_sel[pos] = j0 + i;
                if (out_mass) out_mass[pos] = row[j0 + i];
                ++pos;
            }
            if (eq) ++eq_seen;
        }
    }
}

}  // namespace

hipError_t launch_topk(const TopkParams& p, hipStream_t s) {
    const unsigned blocks = (unsigned)(p.batch * p.num_kv_heads);
    if (blocks == 0) return hipSuccess;
    hipLaunchKernelGGL(topk_kernel, dim3(blocks), dim3(kThreads), 0, s, p);
    return hipGetLastError();
}

}  // namespace locks
