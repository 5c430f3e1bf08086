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
//  1. The 64 groups of 16 consecutive threads (each thread holding pages
//     t, t + 1024, ...) each report their largest key.
//     The k-th largest group maximum T is a real key with at least k keys
//     >= T, so every winner is >= T: a guaranteed lower bound that usually
//     admits only a few dozen candidates.
//  2. Keys >= T are appended to an LDS list (order irrelevant); each
//     candidate's rank is counted against the whole list; rank < k wins
//     (with at most 64 candidates, one wave does this with scalar lane
//     reads instead of LDS loops).
//  3. A winner's output slot is the number of winners with a lower page.
// Fallback (k > 64 or more than kCandCap candidates): bitwise radix select of
// the k-th largest key (one bit per step, counts from wave ballots), then
// two block prefix sums in page order take the keys above it and the
// lowest-page ties.
#include "device_common.hpp"
#include "launchers.hpp"

namespace locks {

namespace {

constexpr int kThreads = 1024;
constexpr int kWaves = kThreads / kWave;
constexpr int kMaxPer = kTopkMaxPages / kThreads;  // keys per thread
constexpr int kFastK = 64;
constexpr int kCandCap = 1024;

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

__global__ __launch_bounds__(kThreads) void topk_kernel(const TopkParams a) {
    __shared__ uint32_t gmax[64];
    __shared__ uint32_t s_thresh;
    __shared__ uint32_t s_ncand;
    __shared__ unsigned long long cand[kCandCap];
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

    // c pages per thread; the fast path holds page j = i*1024 + t in key[i]
    // (coalesced loads; any partition of the pages gives a valid bound), the
    // fallback holds the contiguous pages [t*c, t*c + c) (page-order scans).
    // Loads are unconditional (clamped index, masked) so they are all in
    // flight together; key 0 marks "absent".
    const int c = (n + kThreads - 1) / kThreads;
    uint32_t key[kMaxPer];
    uint32_t my_max = 0;
#pragma unroll
    for (int i = 0; i < kMaxPer; ++i) {
        const int j = i * kThreads + t;
        const float v = row[j < n ? j : n - 1];
        key[i] = (i < c && j < n) ? orderable_bits(v) : 0u;
        my_max = key[i] > my_max ? key[i] : my_max;
    }

    bool fast = k <= kFastK;
    if (fast) {
        const uint32_t gm = umax_in_row(my_max);
        if ((lane & 15) == 0) gmax[wave * 4 + (lane >> 4)] = gm;
        if (t == 0) s_ncand = 0;
        __syncthreads();
        if (wave == 0) {  // k-th largest of the 64 group maxima, bit by bit
            const uint32_t v = gmax[lane];
            uint32_t tau = 0;
            for (int bit = 31; bit >= 0; --bit) {
                const uint32_t cand_t = tau | (1u << bit);
                if (popc64(__ballot(v >= cand_t)) >= (uint32_t)k) tau = cand_t;
            }
            if (lane == 0) s_thresh = tau;
        }
        __syncthreads();
        const uint32_t T = s_thresh;  // >= 1: at least k groups hold a present key
#pragma unroll
        for (int i = 0; i < kMaxPer; ++i) {
            if (i < c && key[i] >= T && key[i] != 0u) {
                const uint32_t slot = atomicAdd(&s_ncand, 1u);
                if (slot < (uint32_t)kCandCap)
                    cand[slot] = ((unsigned long long)key[i] << 32) |
                                 (unsigned long long)(0xffffffffu - (uint32_t)(i * kThreads + t));
            }
        }
        __syncthreads();
        fast = s_ncand <= (uint32_t)kCandCap;  // same value for every thread
    }

    if (fast && s_ncand <= (uint32_t)kWave) {
        // few candidates: one wave ranks them with scalar reads of each lane
        if (wave != 0) return;
        const int C = (int)s_ncand;
        const unsigned long long mine = lane < C ? cand[lane] : 0ull;  // 0 ranks below every key
        const uint32_t lo = (uint32_t)mine, hi = (uint32_t)(mine >> 32);
        int rank = 0;
#pragma unroll
        for (int u = 0; u < kWave; ++u) {
            const uint32_t ulo = __builtin_amdgcn_readlane(lo, u);
            const uint32_t uhi = __builtin_amdgcn_readlane(hi, u);
            const unsigned long long other = ((unsigned long long)uhi << 32) | ulo;
            rank += other > mine ? 1 : 0;
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
            if (out_mass) out_mass[pos] = row[my_page];
        }
        return;
    }
    if (fast) {
        const int C = (int)s_ncand;
        unsigned long long mine = 0;
        bool win = false;
        if (t < C) {
            mine = cand[t];
            int rank = 0;
            for (int u = 0; u < C; ++u) rank += cand[u] > mine ? 1 : 0;
            win = rank < k;
            cand_win[t] = win ? 1 : 0;
        }
        __syncthreads();
        if (win) {
            const uint32_t my_page = 0xffffffffu - (uint32_t)(mine & 0xffffffffu);
            int pos = 0;
            for (int u = 0; u < C; ++u) {
                const uint32_t pu = 0xffffffffu - (uint32_t)(cand[u] & 0xffffffffu);
                pos += (cand_win[u] && pu < my_page) ? 1 : 0;
            }
            out_sel[pos] = (int32_t)my_page;
            if (out_mass) out_mass[pos] = row[my_page];
        }
        return;
    }

    // ---- fallback: exact bitwise search for the k-th largest key, on the
    // contiguous chunk layout
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
