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
//  1. Every thread loads its share of the keys (16-byte loads when the row
//     is aligned).  The 64 groups of 16 consecutive threads each report
//     their largest key.  The k-th largest group maximum T is a real key with
//     at least k keys >= T, so every winner is >= T: a guaranteed lower bound
//     that usually admits only a few dozen candidates.  One wave finds T by
//     ranking the 64 group maxima.
//  2. Keys >= T are compacted per wave (ballot + lane prefix counts) into
//     the wave's own LDS segment; each candidate's rank is counted against
//     the whole list; rank < k wins (with at most 64 candidates, one wave
//     does this with scalar lane reads instead of LDS loops).
//  3. A winner's output slot is the number of winners with a lower page;
//     its mass is recovered from the key, so no second read of the row.
// Run path (k <= 64 and the scan's run maxima given): the same bound is
// taken over the maxima of runs of 16 consecutive pages (each a real key),
// then only the runs whose maximum reaches it are read, one page per
// thread; candidate ranking and output positions are counted by 16 threads
// per candidate with a row reduction.  More than 64 such runs: the fast
// path below.
// Fallback (k > 64 or a wave segment overflows): bitwise radix select of the
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
constexpr int kSeg = kCandCap / kWaves;  // candidate slots per wave

// Inverse of orderable_bits (up to the sign of zero).
__device__ __forceinline__ float key_to_float(uint32_t k) {
    return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

// Flat candidate index i -> slot in the per-wave segments (cnt: per-wave counts).
__device__ __forceinline__ int cand_slot(int i, const uint32_t* cnt) {
    int pre = 0;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
        const int c = (int)cnt[w];
        if (i < pre + c) return w * kSeg + (i - pre);
        pre += c;
    }
    return 0;
}

__device__ __forceinline__ uint32_t popc64(unsigned long long m) { return __popcll(m); }

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

// Top-k over the run maxima, then over the pages of the runs that reach the
// bound.  Returns false (uniformly) when too many runs qualify; nothing has
// been written then.  Each group of 16 consecutive threads (one DPP row)
// handles one list entry i = t / 16 and compares it with entries
// 4 (t % 16) .. +3; the row sum is the entry's count.
__device__ __forceinline__ bool topk_runs(const TopkParams& a, int bg, int n, int k,
                                          const float* row, int32_t* out_sel, float* out_mass,
                                          uint32_t* s_gmax, uint32_t* s_misc,
                                          unsigned long long* s_cand, uint32_t* s_list) {
    constexpr int kMaxRuns = kTopkMaxPages / kRunPages;      // 2048
    constexpr int kRunPer = kMaxRuns / kThreads;             // 2 run maxima per thread
    constexpr int kListCap = kThreads / kRunPages;           // 64 runs read, one page per thread
    const int t = threadIdx.x, wave = t >> 6, lane = t & 63;
    const int i_row = t >> 4, q = t & 15;
    const int nruns_all = (a.max_pages + kRunPages - 1) / kRunPages;
    const int nruns = (n + kRunPages - 1) / kRunPages;  // runs holding present pages
    const float* rm = a.run_max + (size_t)bg * nruns_all;

    uint32_t rkey[kRunPer];
    uint32_t my_max = 0;
#pragma unroll
    for (int i = 0; i < kRunPer; ++i) {
        const int r = i * kThreads + t;
        const float v = rm[r < nruns ? r : nruns - 1];
        rkey[i] = r < nruns ? orderable_bits(v) : 0u;
        my_max = rkey[i] > my_max ? rkey[i] : my_max;
    }
    // 64 group maxima (16 threads each)
    const uint32_t gm = umax_in_row(my_max);
    if (q == 0) s_gmax[i_row] = gm;
    if (t == 0) {
        s_misc[1] = 0;  // qualifying runs
        s_misc[2] = 0;  // candidates
    }
    __syncthreads();
    {  // T = the k-th largest group maximum (ranks by value, then index)
        const uint32_t v = s_gmax[i_row];
        int cnt = 0;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int u = 4 * q + e;
            const uint32_t o = s_gmax[u];
            cnt += (o > v || (o == v && u < i_row)) ? 1 : 0;
        }
        const int rank = (int)sum_in_row((float)cnt);
        if (q == 0 && rank == k - 1) s_misc[0] = v;
    }
    __syncthreads();
    const uint32_t T = s_misc[0];
    // runs whose maximum reaches T (order irrelevant)
#pragma unroll
    for (int i = 0; i < kRunPer; ++i) {
        const bool hit = rkey[i] != 0u && rkey[i] >= T;
        const unsigned long long m = __ballot(hit);
        if (m) {
            uint32_t base = 0;
            if (lane == 0) base = atomicAdd(&s_misc[1], (uint32_t)popc64(m));
            base = __builtin_amdgcn_readfirstlane(base);
            const uint32_t slot = base + __builtin_amdgcn_mbcnt_hi(
                                             (uint32_t)(m >> 32),
                                             __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
            if (hit && slot < (uint32_t)kListCap) s_list[slot] = (uint32_t)(i * kThreads + t);
        }
    }
    __syncthreads();
    const int nlist = (int)s_misc[1];
    if (nlist > kListCap) return false;
    // one page of a listed run per thread; candidates are its keys >= T
    {
        bool hit = false;
        unsigned long long ck = 0;
        if (i_row < nlist) {
            const int j = (int)s_list[i_row] * kRunPages + q;
            if (j < n) {
                const uint32_t key = orderable_bits(row[j]);
                hit = key >= T;
                ck = ((unsigned long long)key << 32) | (unsigned long long)(0xffffffffu - (uint32_t)j);
            }
        }
        const unsigned long long m = __ballot(hit);
        if (m) {
            uint32_t base = 0;
            if (lane == 0) base = atomicAdd(&s_misc[2], (uint32_t)popc64(m));
            base = __builtin_amdgcn_readfirstlane(base);
            const uint32_t slot = base + __builtin_amdgcn_mbcnt_hi(
                                             (uint32_t)(m >> 32),
                                             __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
            if (hit) s_cand[slot] = ck;  // slot < 1024: one candidate per thread at most
        }
    }
    __syncthreads();
    const int C = (int)s_misc[2];  // >= k
    // winners: rank < k; winner of rank r is recorded in s_list[r]
    if (C <= kListCap) {
        const unsigned long long mine = i_row < C ? s_cand[i_row] : 0ull;
        int cnt = 0;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int u = 4 * q + e;
            cnt += (u < C && s_cand[u] > mine) ? 1 : 0;
        }
        const int rank = (int)sum_in_row((float)cnt);
        if (q == 0 && i_row < C && rank < k) s_list[rank] = (uint32_t)i_row;
    } else if (t < C) {  // many candidates (ties at the bound): LDS loops
        const unsigned long long mine = s_cand[t];
        int rank = 0;
        for (int u = 0; u < C; ++u) rank += s_cand[u] > mine ? 1 : 0;
        if (rank < k) s_list[rank] = (uint32_t)t;
    }
    __syncthreads();
    // output slot of winner i_row = winners with a lower page
    if (i_row < k) {
        const unsigned long long mine = s_cand[s_list[i_row]];
        const uint32_t my_page = 0xffffffffu - (uint32_t)mine;
        int cnt = 0;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int u = 4 * q + e;
            const uint32_t pu = u < k ? 0xffffffffu - (uint32_t)s_cand[s_list[u < k ? u : 0]] : 0u;
            cnt += (u < k && pu < my_page) ? 1 : 0;
        }
        const int pos = (int)sum_in_row((float)cnt);
        if (q == 0) {
            out_sel[pos] = (int32_t)my_page;
            if (out_mass) out_mass[pos] = key_to_float((uint32_t)(mine >> 32));
        }
    }
    return true;
}

__global__ __launch_bounds__(kThreads) void topk_kernel(const TopkParams a) {
    __shared__ uint32_t gmax[64];
    __shared__ uint32_t s_thresh;
    __shared__ uint32_t s_cnt[kWaves];
    __shared__ uint32_t s_misc[3];
    __shared__ uint32_t s_list[kFastK];
    __shared__ unsigned long long cand[kCandCap];  // wave w owns [w * kSeg, (w + 1) * kSeg)
    __shared__ unsigned long long flat[kCandCap];
    __shared__ uint8_t cand_win[kCandCap];
    __shared__ uint32_t cnt[3][kWaves];
    __shared__ uint32_t scan_a[kWaves], scan_b[kWaves];

    const int bg = blockIdx.x;
    const int b = bg / a.num_kv_heads;
    const int t = threadIdx.x;
    const int wave = t >> 6;
    const int lane = t & 63;

    int n = a.seq_lens[b] / a.page_size;
    n = n < 0 ? 0 : (n > a.max_pages ? a.max_pages : n);
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

    if (a.run_max && k <= kFastK &&
        topk_runs(a, bg, n, k, row, out_sel, out_mass, gmax, s_misc, cand, s_list))
        return;

    bool fast = k <= kFastK;
    uint32_t key[kMaxPer];
    if (fast) {
        // Any partition of the pages over the threads gives a valid bound.
        // Aligned rows: key slot 4i + e of thread t is page 4(1024 i + t) + e;
        // otherwise page 1024 s + t.  Loads are unconditional (clamped to a
        // vector / page that exists) so they are all in flight together;
        // key 0 marks "absent".
        const bool vec = (reinterpret_cast<uintptr_t>(row) & 15u) == 0 && (a.max_pages & 3) == 0;
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
        auto page_of = [&](int s) {
            return vec ? 4 * ((s >> 2) * kThreads + t) + (s & 3) : s * kThreads + t;
        };

        const uint32_t gm = umax_in_row(my_max);
        if ((lane & 15) == 0) gmax[wave * 4 + (lane >> 4)] = gm;
        __syncthreads();
        if (wave == 0) {
            // rank of each group maximum (larger first, then lower lane): the
            // ranks are a permutation of 0..63, so exactly one lane has rank k-1
            const uint32_t v = gmax[lane];
            int rank = 0;
#pragma unroll
            for (int u = 0; u < kWave; ++u) {
                const uint32_t o = __builtin_amdgcn_readlane(v, u);
                rank += (o > v || (o == v && u < lane)) ? 1 : 0;
            }
            if (rank == k - 1) s_thresh = v;
        }
        __syncthreads();
        const uint32_t T = s_thresh;

        // compaction of the keys >= T into this wave's segment
        uint32_t base = 0;
#pragma unroll
        for (int s = 0; s < kMaxPer; ++s) {
            const bool is_c = key[s] != 0u && key[s] >= T;
            const unsigned long long m = __ballot(is_c);
            if (m) {
                const uint32_t below = __builtin_amdgcn_mbcnt_hi(
                    (uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
                const uint32_t slot = base + below;
                if (is_c && slot < (uint32_t)kSeg)
                    cand[wave * kSeg + slot] =
                        ((unsigned long long)key[s] << 32) |
                        (unsigned long long)(0xffffffffu - (uint32_t)page_of(s));
                base += (uint32_t)popc64(m);
            }
        }
        if (lane == 0) s_cnt[wave] = base;
        __syncthreads();
        int C = 0;
#pragma unroll
        for (int w2 = 0; w2 < kWaves; ++w2) {
            const uint32_t cw = s_cnt[w2];
            C += (int)cw;
            fast = fast && cw <= (uint32_t)kSeg;  // same value for every thread
        }

        if (fast && C <= kWave) {
            // few candidates: one wave ranks them with scalar reads of each lane
            if (wave != 0) return;
            const unsigned long long mine = lane < C ? cand[cand_slot(lane, s_cnt)] : 0ull;
            const uint32_t lo = (uint32_t)mine, hi = (uint32_t)(mine >> 32);
            int rank = 0;
#pragma unroll
            for (int u = 0; u < kWave; ++u) {
                const uint32_t ulo = __builtin_amdgcn_readlane(lo, u);
                const uint32_t uhi = __builtin_amdgcn_readlane(hi, u);
                const unsigned long long other = ((unsigned long long)uhi << 32) | ulo;
                rank += other > mine ? 1 : 0;  // 0 (absent lanes) ranks below every key
            }
            const bool win = lane < C && rank < k;
            const uint32_t my_page = 0xffffffffu - lo;
            const unsigned long long wins = __ballot(win);
            int pos = 0;
#pragma unroll
            for (int u = 0; u < kWave; ++u) {
                const uint32_t pu = __builtin_amdgcn_readlane(my_page, u);
                pos += (((wins >> u) & 1ull) && pu < my_page) ? 1 : 0;
            }
            if (win) {
                out_sel[pos] = (int32_t)my_page;
                if (out_mass) out_mass[pos] = key_to_float(hi);
            }
            return;
        }
        if (fast) {
            if (t < C) flat[t] = cand[cand_slot(t, s_cnt)];
            __syncthreads();
            unsigned long long mine = 0;
            bool win = false;
            if (t < C) {
                mine = flat[t];
                int rank = 0;
                for (int u = 0; u < C; ++u) rank += flat[u] > mine ? 1 : 0;
                win = rank < k;
                cand_win[t] = win ? 1 : 0;
            }
            __syncthreads();
            if (win) {
                const uint32_t my_page = 0xffffffffu - (uint32_t)(mine & 0xffffffffu);
                int pos = 0;
                for (int u = 0; u < C; ++u) {
                    const uint32_t pu = 0xffffffffu - (uint32_t)(flat[u] & 0xffffffffu);
                    pos += (cand_win[u] && pu < my_page) ? 1 : 0;
                }
                out_sel[pos] = (int32_t)my_page;
                if (out_mass) out_mass[pos] = key_to_float((uint32_t)(mine >> 32));
            }
            return;
        }
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
