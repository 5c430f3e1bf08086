// Mean-of-share group score (gist.science technical summary, section 2,
// Group-Shared Selection: the query heads' estimated mass shares are
// averaged over the group into one selection table).  From per-head
// estimates s[b][h][j] (natural log, -inf for pages that are not full):
//   Z[b][h]          = log sum over full pages j of exp(s[b][h][j])
//   score[b][g][j]   = log( (1/G) sum_{h in g} exp(s[b][h][j] - Z[b][h]) )
// Two kernels: one workgroup reduces each (b, h) row to Z; then one thread
// per (b, g, page) forms the score, and each row of 16 threads (one run of
// 16 pages) writes the run maximum for the top-k.
#include "device_common.hpp"
#include "launchers.hpp"

namespace locks {

namespace {

constexpr int kShareThreads = 256;

// Z for one (b, h).  Per chunk of 64 x 256 pages every thread issues its 64
// strided loads at once, takes their maximum, then sums 2^(x - max) (one
// exp2 per page); chunks and then waves are combined as (max, sum) pairs
// (log2 units).
constexpr int kShareVals = 64;  // pages per thread and chunk
__global__ __launch_bounds__(kShareThreads) void head_total_kernel(const ShareParams a) {
    __shared__ float sm_m[kShareThreads / kWave], sm_s[kShareThreads / kWave];
    const int bh = blockIdx.x;
    const int b = bh / a.num_q_heads;
    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    const int full = candidate_pages(a.seq_lens[b], a.summarized ? a.summarized[b] : 0,
                                     a.summarized != nullptr, a.page_size, a.max_pages);
    const float* row = a.head_logmass + (size_t)bh * a.max_pages;
    float m = -INFINITY, sum = 0.f;
    for (int base = 0; base < full; base += kShareThreads * kShareVals) {
        float x[kShareVals];
#pragma unroll
        for (int e = 0; e < kShareVals; ++e) {
            const int j = base + t + kShareThreads * e;
            const float v = row[j < full ? j : 0];  // in-bounds address either way
            x[e] = j < full ? v * kLog2e : -INFINITY;
        }
        float cm = -INFINITY;
#pragma unroll
        for (int e = 0; e < kShareVals; ++e) cm = fmaxf(cm, x[e]);
        if (cm != -INFINITY) {
            float cs = 0.f;
#pragma unroll
            for (int e = 0; e < kShareVals; ++e) cs += fast_exp2(x[e] - cm);
            const float mn = fmaxf(m, cm);
            sum = (m == -INFINITY ? 0.f : sum * fast_exp2(m - mn)) + cs * fast_exp2(cm - mn);
            m = mn;
        }
    }
    const float wm = wave_max(m);
    float ws = wm == -INFINITY ? 0.f : sum * fast_exp2(m - wm);
    ws = wave_sum(ws);
    if (lane == 0) {
        sm_m[wave] = wm;
        sm_s[wave] = ws;
    }
    __syncthreads();
    if (t == 0) {
        float M = -INFINITY;
        for (int w2 = 0; w2 < kShareThreads / kWave; ++w2) M = fmaxf(M, sm_m[w2]);
        float S = 0.f;
        if (M != -INFINITY)
            for (int w2 = 0; w2 < kShareThreads / kWave; ++w2)
                S += sm_m[w2] == -INFINITY ? 0.f : sm_s[w2] * fast_exp2(sm_m[w2] - M);
        a.head_total[bh] = S > 0.f ? (M + fast_log2(S)) * kLn2 : -INFINITY;
    }
}

// One thread per (b, g, page j).
__global__ __launch_bounds__(kShareThreads) void share_kernel(const ShareParams a) {
    const int Hkv = a.num_kv_heads, G = a.num_q_heads / Hkv;
    const int nchunk = (a.max_pages + kShareThreads - 1) / kShareThreads;
    const int bg = blockIdx.x / nchunk;
    const int b = bg / Hkv, g = bg % Hkv;
    const int j = (blockIdx.x % nchunk) * kShareThreads + threadIdx.x;
    const int full = candidate_pages(a.seq_lens[b], a.summarized ? a.summarized[b] : 0,
                                     a.summarized != nullptr, a.page_size, a.max_pages);
    float score = -INFINITY;
    if (j < full) {
        const float* hm = a.head_logmass + ((size_t)b * a.num_q_heads + g * G) * a.max_pages + j;
        const float* z = a.head_total + (size_t)b * a.num_q_heads + g * G;
        float x[16];  // G <= 16; fully unrolled so the array stays in registers
        float mx = -INFINITY;
#pragma unroll
        for (int hh = 0; hh < 16; ++hh) {
            x[hh] = hh < G ? (hm[(size_t)(hh < G ? hh : 0) * a.max_pages] - z[hh < G ? hh : 0]) * kLog2e
                           : -INFINITY;
            mx = fmaxf(mx, x[hh]);
        }
        if (mx != -INFINITY) {
            float s = 0.f;
#pragma unroll
            for (int hh = 0; hh < 16; ++hh) s += hh < G ? fast_exp2(x[hh] - mx) : 0.f;
            score = (mx + fast_log2(s / (float)G)) * kLn2;
        }
    }
    if (j < a.max_pages) a.page_logmass[(size_t)bg * a.max_pages + j] = score;
    if (a.run_max) {
        // rows of 16 threads are runs of 16 pages (the chunk size is a multiple of 16)
        const float rm = max_in_row(score);
        const int nruns = (a.max_pages + kRunPages - 1) / kRunPages;
        if ((threadIdx.x & 15) == 0 && j < a.max_pages)
            a.run_max[(size_t)bg * nruns + j / kRunPages] = rm;
    }
}

}  // namespace

hipError_t launch_share(const ShareParams& p, hipStream_t s) {
    static_assert(kShareThreads % kRunPages == 0 && kRunPages == 16, "runs are DPP rows");
    const unsigned rows = (unsigned)(p.batch * p.num_q_heads);
    if (rows == 0) return hipSuccess;
    hipLaunchKernelGGL(head_total_kernel, dim3(rows), dim3(kShareThreads), 0, s, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int nchunk = (p.max_pages + kShareThreads - 1) / kShareThreads;
    const unsigned blocks = (unsigned)(p.batch * p.num_kv_heads * nchunk);
    hipLaunchKernelGGL(share_kernel, dim3(blocks), dim3(kShareThreads), 0, s, p);
    return hipGetLastError();
}

}  // namespace locks
