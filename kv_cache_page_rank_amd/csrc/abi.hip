// C ABI of the library (declared in include/locks.h): host-side validation,
// workspace sizing, dispatch to the kernel launchers and graph capture.
// Nothing here allocates device memory; nothing here reads device memory.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <mutex>
#include <new>

#include "../../include/locks.h"
#include "launchers.hpp"

namespace {

thread_local int32_t g_last_hip_error = 0;

locks_status hip_fail(hipError_t e) {
    g_last_hip_error = (int32_t)e;
    return LOCKS_ERR_HIP;
}

constexpr size_t kAlign = 256;
size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

bool head_dims_ok(int32_t hq, int32_t hkv) {
    return hq > 0 && hkv > 0 && hq % hkv == 0 && hq / hkv <= 16;
}

locks_status check_page_table(const locks_page_table* pt) {
    if (!pt || !pt->block_table || !pt->seq_lens || pt->batch <= 0 || pt->max_pages <= 0)
        return LOCKS_ERR_INVALID_ARG;
    if (pt->max_pages > locks::kTopkMaxPages) return LOCKS_ERR_UNSUPPORTED;
    return LOCKS_OK;
}

static_assert((int)LOCKS_F32 == (int)locks::kSummF32 && (int)LOCKS_BF16 == (int)locks::kSummBF16 &&
                  (int)LOCKS_Q8Q4 == (int)locks::kSummQ8Q4,
              "summary dtypes are passed through to the kernels");

locks_status check_summaries(const locks_summaries* s, bool need_data) {
    if (!s || s->num_blocks <= 0 || s->num_kv_heads <= 0 || s->page_size <= 0 ||
        s->head_dim <= 0 || s->rank <= 0)
        return LOCKS_ERR_INVALID_ARG;
    if (s->dtype != LOCKS_F32 && s->dtype != LOCKS_BF16 && s->dtype != LOCKS_Q8Q4)
        return LOCKS_ERR_INVALID_ARG;
    if (need_data && (!s->mu || !s->basis || !s->coef)) return LOCKS_ERR_INVALID_ARG;
    if (need_data && s->dtype == LOCKS_Q8Q4 && !s->scales) return LOCKS_ERR_INVALID_ARG;
    if (!locks::scan_supported(s->page_size, s->head_dim, s->rank)) return LOCKS_ERR_UNSUPPORTED;
    return LOCKS_OK;
}

locks_status check_cache(const locks_kv_cache* kv, bool need_v) {
    if (!kv || !kv->k || (need_v && !kv->v) || kv->num_blocks <= 0 || kv->num_kv_heads <= 0 ||
        kv->page_size <= 0 || kv->head_dim <= 0)
        return LOCKS_ERR_INVALID_ARG;
    if (kv->dtype != LOCKS_F32 && kv->dtype != LOCKS_BF16) return LOCKS_ERR_INVALID_ARG;
    return LOCKS_OK;
}

int32_t num_runs(int32_t max_pages) { return (max_pages + locks::kRunPages - 1) / locks::kRunPages; }

// Selection workspace: page masses, run maxima, per-head estimates and
// per-head totals (the last two for the mean-of-share aggregation).
size_t select_mass_bytes(int32_t batch, int32_t max_pages, int32_t hkv) {
    return align_up((size_t)batch * hkv * max_pages * sizeof(float));
}
size_t select_run_bytes(int32_t batch, int32_t max_pages, int32_t hkv) {
    return align_up((size_t)batch * hkv * num_runs(max_pages) * sizeof(float));
}
size_t select_head_bytes(int32_t batch, int32_t max_pages, int32_t hq) {
    return align_up((size_t)batch * hq * max_pages * sizeof(float));
}
size_t total_bytes(int32_t batch, int32_t hq) { return align_up((size_t)batch * hq * sizeof(float)); }
size_t select_ws(int32_t batch, int32_t max_pages, int32_t hq, int32_t hkv) {
    return select_mass_bytes(batch, max_pages, hkv) + select_run_bytes(batch, max_pages, hkv) +
           select_head_bytes(batch, max_pages, hq) + total_bytes(batch, hq);
}

size_t attend_ws(int32_t batch, int32_t hq, int32_t d, int32_t splits) {
    const size_t rows = (size_t)batch * hq * splits;
    return align_up(rows * 2 * sizeof(float)) + align_up(rows * d * sizeof(float));
}

int32_t dense_splits(int32_t batch, int32_t hkv, int32_t max_pages) {
    const int pps = locks::dense_pages_per_split(batch, hkv, max_pages);
    return (max_pages + pps - 1) / pps;
}

// Shared body of the attention entry points.
locks_status attend_common(const float* q, int32_t hq, const locks_kv_cache* kv,
                           const locks_page_table* pt, const int32_t* sel, int32_t k_pages,
                           void* out, float* out_lse, void* ws, size_t ws_bytes,
                           hipStream_t stream) {
    locks_status st = check_cache(kv, true);
    if (st != LOCKS_OK) return st;
    if ((st = check_page_table(pt)) != LOCKS_OK) return st;
    if (!q || !out || !head_dims_ok(hq, kv->num_kv_heads)) return LOCKS_ERR_INVALID_ARG;
    const bool sparse = sel != nullptr;
    if (sparse && k_pages < 0) return LOCKS_ERR_INVALID_ARG;
    if (!locks::attend_supported(kv->dtype == LOCKS_BF16, kv->page_size, kv->head_dim))
        return LOCKS_ERR_UNSUPPORTED;
    const int32_t splits = sparse ? k_pages + 1 : dense_splits(pt->batch, kv->num_kv_heads, pt->max_pages);
    const size_t need = attend_ws(pt->batch, hq, kv->head_dim, splits);
    if (!ws || ws_bytes < need) return LOCKS_ERR_WORKSPACE;
    locks::AttnParams p{};
    p.q = q;
    p.k = kv->k;
    p.v = kv->v;
    p.bf16 = kv->dtype == LOCKS_BF16;
    p.block_table = pt->block_table;
    p.seq_lens = pt->seq_lens;
    p.summarized = pt->summarized;
    p.sel_pages = sel;
    p.batch = pt->batch;
    p.num_q_heads = hq;
    p.num_kv_heads = kv->num_kv_heads;
    p.max_pages = pt->max_pages;
    p.num_blocks = kv->num_blocks;
    p.page_size = kv->page_size;
    p.head_dim = kv->head_dim;
    p.k_sel = sparse ? k_pages : 0;
    p.pages_per_split = sparse ? 1 : locks::dense_pages_per_split(pt->batch, kv->num_kv_heads, pt->max_pages);
    p.num_splits = splits;
    const size_t rows = (size_t)pt->batch * hq * splits;
    p.part_ml = static_cast<float*>(ws);
    p.part_o = reinterpret_cast<float*>(static_cast<char*>(ws) + align_up(rows * 2 * sizeof(float)));
    p.out = out;
    p.out_lse = out_lse;
    const hipError_t e = locks::launch_attend(p, stream);
    return e == hipSuccess ? LOCKS_OK : hip_fail(e);
}

locks_status scan_common(const float* q, int32_t hq, const locks_summaries* s,
                         const locks_page_table* pt, float* page_logmass, float* head_logmass,
                         float* run_max, hipStream_t stream) {
    locks::ScanParams p{};
    p.q = q;
    p.mu = s->mu;
    p.basis = s->basis;
    p.coef = s->coef;
    p.summ_dtype = s->dtype;  // locks_dtype values match locks::SummDtype
    p.scales = s->scales;
    p.block_table = pt->block_table;
    p.seq_lens = pt->seq_lens;
    p.summarized = pt->summarized;
    p.batch = pt->batch;
    p.num_q_heads = hq;
    p.num_kv_heads = s->num_kv_heads;
    p.max_pages = pt->max_pages;
    p.num_blocks = s->num_blocks;
    p.page_size = s->page_size;
    p.head_dim = s->head_dim;
    p.rank = s->rank;
    p.page_logmass = page_logmass;
    p.head_logmass = head_logmass;
    p.run_max = run_max;
    const hipError_t e = locks::launch_scan(p, stream);
    return e == hipSuccess ? LOCKS_OK : hip_fail(e);
}

locks_status topk_common(const float* page_logmass, const locks_page_table* pt, int32_t hkv,
                         int32_t page_size, int32_t budget, int32_t width, int32_t* sel,
                         float* sel_mass, const float* run_max, hipStream_t stream) {
    locks::TopkParams p{};
    p.page_logmass = page_logmass;
    p.seq_lens = pt->seq_lens;
    p.summarized = pt->summarized;
    p.batch = pt->batch;
    p.num_kv_heads = hkv;
    p.max_pages = pt->max_pages;
    p.page_size = page_size;
    const int32_t k = budget / page_size;
    p.k_req = k < width ? k : width;
    p.width = width;
    p.sel_pages = sel;
    p.sel_logmass = sel_mass;
    p.run_max = run_max;
    const hipError_t e = locks::launch_topk(p, stream);
    return e == hipSuccess ? LOCKS_OK : hip_fail(e);
}

locks_status share_common(const float* head_logmass, int32_t hq, int32_t hkv,
                          const locks_page_table* pt, int32_t page_size, float* head_total,
                          float* page_logmass, float* run_max, hipStream_t stream) {
    locks::ShareParams p{};
    p.head_logmass = head_logmass;
    p.seq_lens = pt->seq_lens;
    p.summarized = pt->summarized;
    p.batch = pt->batch;
    p.num_q_heads = hq;
    p.num_kv_heads = hkv;
    p.max_pages = pt->max_pages;
    p.page_size = page_size;
    p.head_total = head_total;
    p.page_logmass = page_logmass;
    p.run_max = run_max;
    const hipError_t e = locks::launch_share(p, stream);
    return e == hipSuccess ? LOCKS_OK : hip_fail(e);
}

}  // namespace

struct locks_step_graph {
    hipGraphExec_t exec;
};

extern "C" {

size_t locks_workspace_bytes(int32_t op, int32_t batch, int32_t max_pages, int32_t num_q_heads,
                             int32_t num_kv_heads, int32_t page_size, int32_t head_dim,
                             int32_t rank, int32_t k_pages) {
    (void)page_size;
    (void)rank;
    if (batch <= 0 || max_pages <= 0 || num_q_heads <= 0 || num_kv_heads <= 0 || head_dim <= 0)
        return 0;
    switch (op) {
        case LOCKS_OP_BUILD:
            return 0;
        case LOCKS_OP_SELECT:
            return select_ws(batch, max_pages, num_q_heads, num_kv_heads);
        case LOCKS_OP_SPARSE_ATTEND:
            return attend_ws(batch, num_q_heads, head_dim, (k_pages < 0 ? 0 : k_pages) + 1);
        case LOCKS_OP_DENSE_ATTEND:
            return attend_ws(batch, num_q_heads, head_dim, dense_splits(batch, num_kv_heads, max_pages));
        case LOCKS_OP_STEP:
            return select_ws(batch, max_pages, num_q_heads, num_kv_heads) +
                   attend_ws(batch, num_q_heads, head_dim, (k_pages < 0 ? 0 : k_pages) + 1);
        default:
            return 0;
    }
}

namespace {

locks_status build_common(const locks_kv_cache* cache, const locks_page_table* pages,
                          const int32_t* page_begin, int32_t refresh_pages,
                          const locks_summaries* out, hipStream_t stream) {
    locks_status st = check_cache(cache, false);
    if (st != LOCKS_OK) return st;
    if ((st = check_page_table(pages)) != LOCKS_OK) return st;
    if ((st = check_summaries(out, true)) != LOCKS_OK) return st;
    if (out->num_blocks != cache->num_blocks || out->num_kv_heads != cache->num_kv_heads ||
        out->page_size != cache->page_size || out->head_dim != cache->head_dim)
        return LOCKS_ERR_INVALID_ARG;
    if (!locks::build_supported(cache->page_size, cache->head_dim, out->rank))
        return LOCKS_ERR_UNSUPPORTED;
    locks::BuildParams p{};
    p.k = cache->k;
    p.bf16 = cache->dtype == LOCKS_BF16;
    p.block_table = pages->block_table;
    p.seq_lens = pages->seq_lens;
    p.page_begin = page_begin;
    p.refresh_pages = refresh_pages;
    p.batch = pages->batch;
    p.num_kv_heads = cache->num_kv_heads;
    p.max_pages = pages->max_pages;
    p.num_blocks = cache->num_blocks;
    p.page_size = cache->page_size;
    p.head_dim = cache->head_dim;
    p.rank = out->rank;
    p.mu = out->mu;
    p.basis = out->basis;
    p.coef = out->coef;
    p.out_dtype = out->dtype;
    p.scales = out->scales;
    const hipError_t e = locks::launch_build(p, stream);
    return e == hipSuccess ? LOCKS_OK : hip_fail(e);
}

}  // namespace

locks_status locks_build_sketch_summaries(const locks_kv_cache* cache,
                                          const locks_page_table* pages,
                                          const int32_t* page_begin, const float* shared_basis,
                                          const locks_summaries* out, void* stream) {
    locks_status st = check_cache(cache, false);
    if (st != LOCKS_OK) return st;
    if ((st = check_page_table(pages)) != LOCKS_OK) return st;
    if ((st = check_summaries(out, true)) != LOCKS_OK) return st;
    if (!shared_basis || out->dtype != LOCKS_F32 || out->num_blocks != cache->num_blocks ||
        out->num_kv_heads != cache->num_kv_heads || out->page_size != cache->page_size ||
        out->head_dim != cache->head_dim)
        return LOCKS_ERR_INVALID_ARG;
    if (!locks::build_supported(cache->page_size, cache->head_dim, out->rank))
        return LOCKS_ERR_UNSUPPORTED;
    locks::BuildParams p{};
    p.k = cache->k;
    p.bf16 = cache->dtype == LOCKS_BF16;
    p.block_table = pages->block_table;
    p.seq_lens = pages->seq_lens;
    p.page_begin = page_begin;
    p.batch = pages->batch;
    p.num_kv_heads = cache->num_kv_heads;
    p.max_pages = pages->max_pages;
    p.num_blocks = cache->num_blocks;
    p.page_size = cache->page_size;
    p.head_dim = cache->head_dim;
    p.rank = out->rank;
    p.mu = out->mu;
    p.basis = out->basis;
    p.coef = out->coef;
    p.out_dtype = out->dtype;
    const hipError_t e = locks::launch_sketch(p, shared_basis, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? LOCKS_OK : hip_fail(e);
}

locks_status locks_build_summaries(const locks_kv_cache* cache, const locks_page_table* pages,
                                   const int32_t* page_begin, const locks_summaries* out,
                                   void* ws, size_t ws_bytes, void* stream) {
    (void)ws;
    (void)ws_bytes;
    return build_common(cache, pages, page_begin, 0, out, static_cast<hipStream_t>(stream));
}

locks_status locks_refresh_summaries(const locks_kv_cache* cache, const locks_page_table* pages,
                                     const int32_t* page_begin, int32_t max_new_pages,
                                     const locks_summaries* out, void* stream) {
    if (!page_begin || max_new_pages <= 0) return LOCKS_ERR_INVALID_ARG;
    hipStream_t s = static_cast<hipStream_t>(stream);
    const locks_status st = build_common(cache, pages, page_begin, max_new_pages, out, s);
    if (st != LOCKS_OK || !pages->summarized) return st;
    // the new summaries exist once the build above is done (stream order):
    // the count advances after it
    const hipError_t e = locks::launch_advance_summarized(
        pages->seq_lens, page_begin, pages->summarized, pages->batch, cache->page_size,
        pages->max_pages, max_new_pages, s);
    return e == hipSuccess ? LOCKS_OK : hip_fail(e);
}

locks_status locks_quantize_summaries(const locks_summaries* src, const locks_summaries* dst,
                                      void* stream) {
    locks_status st = check_summaries(src, true);
    if (st != LOCKS_OK) return st;
    if ((st = check_summaries(dst, true)) != LOCKS_OK) return st;
    if (src->dtype != LOCKS_F32 || dst->dtype != LOCKS_Q8Q4 ||
        src->num_blocks != dst->num_blocks || src->num_kv_heads != dst->num_kv_heads ||
        src->page_size != dst->page_size || src->head_dim != dst->head_dim ||
        src->rank != dst->rank)
        return LOCKS_ERR_INVALID_ARG;
    locks::QuantParams p{};
    p.mu = static_cast<const float*>(src->mu);
    p.basis = static_cast<const float*>(src->basis);
    p.coef = static_cast<const float*>(src->coef);
    p.mu_q = static_cast<int8_t*>(dst->mu);
    p.basis_q = static_cast<uint8_t*>(dst->basis);
    p.coef_q = static_cast<int8_t*>(dst->coef);
    p.scales = dst->scales;
    p.units = (int64_t)src->num_blocks * src->num_kv_heads;
    p.page_size = src->page_size;
    p.head_dim = src->head_dim;
    p.rank = src->rank;
    const hipError_t e = locks::launch_quantize(p, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? LOCKS_OK : hip_fail(e);
}

locks_status locks_scan(const float* q, int32_t num_q_heads, const locks_summaries* summaries,
                        const locks_page_table* pages, float* page_logmass, float* head_logmass,
                        float* run_max, void* stream) {
    locks_status st = check_summaries(summaries, true);
    if (st != LOCKS_OK) return st;
    if ((st = check_page_table(pages)) != LOCKS_OK) return st;
    if (!q || !page_logmass || !head_dims_ok(num_q_heads, summaries->num_kv_heads))
        return LOCKS_ERR_INVALID_ARG;
    return scan_common(q, num_q_heads, summaries, pages, page_logmass, head_logmass, run_max,
                       static_cast<hipStream_t>(stream));
}

locks_status locks_topk(const float* page_logmass, const locks_page_table* pages,
                        int32_t num_kv_heads, int32_t page_size, int32_t budget_tokens,
                        int32_t width, int32_t* sel_pages, float* sel_logmass,
                        const float* run_max, void* stream) {
    locks_status st = check_page_table(pages);
    if (st != LOCKS_OK) return st;
    if (!page_logmass || !sel_pages || num_kv_heads <= 0 || page_size <= 0 || budget_tokens < 0 ||
        width < 0)
        return LOCKS_ERR_INVALID_ARG;
    if (width == 0) return LOCKS_OK;
    return topk_common(page_logmass, pages, num_kv_heads, page_size, budget_tokens, width,
                       sel_pages, sel_logmass, run_max, static_cast<hipStream_t>(stream));
}

locks_status locks_select(const float* q, int32_t num_q_heads, const locks_summaries* summaries,
                          const locks_page_table* pages, int32_t budget_tokens, int32_t agg,
                          int32_t* sel_pages, float* sel_logmass, float* page_logmass, void* ws,
                          size_t ws_bytes, void* stream) {
    locks_status st = check_summaries(summaries, true);
    if (st != LOCKS_OK) return st;
    if ((st = check_page_table(pages)) != LOCKS_OK) return st;
    if (!q || budget_tokens < 0 || !head_dims_ok(num_q_heads, summaries->num_kv_heads))
        return LOCKS_ERR_INVALID_ARG;
    if (agg != LOCKS_AGG_LSE && agg != LOCKS_AGG_MEAN_SHARE) return LOCKS_ERR_INVALID_ARG;
    const int32_t width = budget_tokens / summaries->page_size;
    if (width > 0 && !sel_pages) return LOCKS_ERR_INVALID_ARG;
    // The workspace holds the page masses (unless the caller takes them), the
    // run maxima and, for the mean-of-share aggregation, the per-head
    // estimates and totals; without a workspace (LSE only) the top-k reads
    // every mass.
    const int32_t B = pages->batch, MP = pages->max_pages, hkv = summaries->num_kv_heads;
    const bool have_ws = ws && ws_bytes >= select_ws(B, MP, num_q_heads, hkv);
    if (agg == LOCKS_AGG_MEAN_SHARE && !have_ws) return LOCKS_ERR_WORKSPACE;
    float* masses = page_logmass;
    if (!masses) {
        if (!have_ws) return LOCKS_ERR_WORKSPACE;
        masses = static_cast<float*>(ws);
    }
    char* wsb = static_cast<char*>(ws);
    float* run_max =
        have_ws ? reinterpret_cast<float*>(wsb + select_mass_bytes(B, MP, hkv)) : nullptr;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (agg == LOCKS_AGG_MEAN_SHARE) {
        const size_t heads_off = select_mass_bytes(B, MP, hkv) + select_run_bytes(B, MP, hkv);
        float* heads = reinterpret_cast<float*>(wsb + heads_off);
        float* totals =
            reinterpret_cast<float*>(wsb + heads_off + select_head_bytes(B, MP, num_q_heads));
        if ((st = scan_common(q, num_q_heads, summaries, pages, masses, heads, nullptr, s)) !=
            LOCKS_OK)
            return st;
        if ((st = share_common(heads, num_q_heads, hkv, pages, summaries->page_size, totals,
                               masses, run_max, s)) != LOCKS_OK)
            return st;
    } else if ((st = scan_common(q, num_q_heads, summaries, pages, masses, nullptr, run_max, s)) !=
               LOCKS_OK) {
        return st;
    }
    if (width == 0) return LOCKS_OK;
    return topk_common(masses, pages, summaries->num_kv_heads, summaries->page_size, budget_tokens,
                       width, sel_pages, sel_logmass, run_max, s);
}

locks_status locks_mean_share(const float* head_logmass, int32_t num_q_heads,
                              int32_t num_kv_heads, const locks_page_table* pages,
                              int32_t page_size, float* page_logmass, float* run_max, void* ws,
                              size_t ws_bytes, void* stream) {
    locks_status st = check_page_table(pages);
    if (st != LOCKS_OK) return st;
    if (!head_logmass || !page_logmass || page_size <= 0 || !head_dims_ok(num_q_heads, num_kv_heads))
        return LOCKS_ERR_INVALID_ARG;
    if (!ws || ws_bytes < total_bytes(pages->batch, num_q_heads)) return LOCKS_ERR_WORKSPACE;
    return share_common(head_logmass, num_q_heads, num_kv_heads, pages, page_size,
                        static_cast<float*>(ws), page_logmass, run_max,
                        static_cast<hipStream_t>(stream));
}

}  // extern "C"

// Scratch of locks_select_noalloc: the selection workspace (page masses, run
// maxima, per-head estimates and totals) in a static device array, so that
// entry point never allocates.  Each device holds its own copy; its address
// is looked up once per device (hipGetSymbolAddress, with that device
// current) and kept.  In host code `scratch` itself is only a stand-in for
// the symbol: kernels get the looked-up address, never the name.
namespace {

constexpr size_t kNoAllocScratchBytes = size_t(16) << 20;
static __device__ __align__(256) char scratch[kNoAllocScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices] = {};

locks_status scratch_of_current_device(void** out) {
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e);
    if (dev < 0 || dev >= kMaxDevices) return LOCKS_ERR_UNSUPPORTED;
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (!g_scratch_ptr[dev]) {
        void* ptr = nullptr;
        e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return hip_fail(e);
        if (!ptr) return hip_fail(hipErrorInvalidSymbol);
        g_scratch_ptr[dev] = ptr;
    }
    *out = g_scratch_ptr[dev];
    return LOCKS_OK;
}

}  // namespace

extern "C" {

locks_status locks_select_noalloc(const float* q, int32_t num_q_heads,
                                  const locks_summaries* summaries, const locks_page_table* pages,
                                  int32_t budget_tokens, int32_t agg, int32_t* sel_pages,
                                  float* sel_logmass, float* page_logmass, void* stream) {
    locks_status st = check_summaries(summaries, true);
    if (st != LOCKS_OK) return st;
    if ((st = check_page_table(pages)) != LOCKS_OK) return st;
    if (!q || budget_tokens < 0 || !head_dims_ok(num_q_heads, summaries->num_kv_heads))
        return LOCKS_ERR_INVALID_ARG;
    const size_t need =
        select_ws(pages->batch, pages->max_pages, num_q_heads, summaries->num_kv_heads);
    if (need > kNoAllocScratchBytes) return LOCKS_ERR_WORKSPACE;
    void* ws = nullptr;
    if ((st = scratch_of_current_device(&ws)) != LOCKS_OK) return st;
    return locks_select(q, num_q_heads, summaries, pages, budget_tokens, agg, sel_pages,
                        sel_logmass, page_logmass, ws, need, stream);
}

locks_status locks_sparse_attend(const float* q, int32_t num_q_heads, const locks_kv_cache* cache,
                                 const locks_page_table* pages, const int32_t* sel_pages,
                                 int32_t k_pages, void* out, float* out_lse, void* ws,
                                 size_t ws_bytes, void* stream) {
    if (k_pages > 0 && !sel_pages) return LOCKS_ERR_INVALID_ARG;
    // With k_pages == 0 the sparse path still attends the partial last page;
    // a non-null marker selects that path.  The marker is a device array (the
    // sequence lengths) because the kernels read a list entry before they
    // know whether they use it; with k_pages == 0 they never use it.
    const int32_t* sel = k_pages > 0 ? sel_pages : pages->seq_lens;
    return attend_common(q, num_q_heads, cache, pages, sel, k_pages, out, out_lse, ws, ws_bytes,
                         static_cast<hipStream_t>(stream));
}

locks_status locks_dense_attend(const float* q, int32_t num_q_heads, const locks_kv_cache* cache,
                                const locks_page_table* pages, void* out, float* out_lse,
                                void* ws, size_t ws_bytes, void* stream) {
    return attend_common(q, num_q_heads, cache, pages, nullptr, 0, out, out_lse, ws, ws_bytes,
                         static_cast<hipStream_t>(stream));
}

locks_status locks_step_graph_create(const locks_step_args* a, locks_step_graph** graph) {
    if (!a || !graph) return LOCKS_ERR_INVALID_ARG;
    *graph = nullptr;
    const int32_t k = a->summaries.page_size > 0 ? a->budget_tokens / a->summaries.page_size : 0;
    const size_t sel_bytes =
        select_ws(a->pages.batch, a->pages.max_pages, a->num_q_heads, a->summaries.num_kv_heads);
    const size_t need = locks_workspace_bytes(LOCKS_OP_STEP, a->pages.batch, a->pages.max_pages,
                                              a->num_q_heads, a->summaries.num_kv_heads,
                                              a->summaries.page_size, a->summaries.head_dim,
                                              a->summaries.rank, k);
    if (!a->ws || a->ws_bytes < need) return LOCKS_ERR_WORKSPACE;
    if (a->cache.page_size != a->summaries.page_size || a->cache.head_dim != a->summaries.head_dim ||
        a->cache.num_kv_heads != a->summaries.num_kv_heads)
        return LOCKS_ERR_INVALID_ARG;

    hipStream_t s;
    hipError_t e = hipStreamCreateWithFlags(&s, hipStreamNonBlocking);
    if (e != hipSuccess) return hip_fail(e);
    e = hipStreamBeginCapture(s, hipStreamCaptureModeThreadLocal);
    if (e != hipSuccess) {
        (void)hipStreamDestroy(s);
        return hip_fail(e);
    }
    locks_status st = locks_select(a->q, a->num_q_heads, &a->summaries, &a->pages,
                                   a->budget_tokens, a->agg, a->sel_pages, a->sel_logmass,
                                   a->page_logmass, a->ws, a->ws_bytes, s);
    if (st == LOCKS_OK) {
        void* attn_ws = static_cast<char*>(a->ws) + sel_bytes;
        st = locks_sparse_attend(a->q, a->num_q_heads, &a->cache, &a->pages, a->sel_pages, k, a->out,
                                 a->out_lse, attn_ws, a->ws_bytes - sel_bytes, s);
    }
    hipGraph_t g = nullptr;
    e = hipStreamEndCapture(s, &g);
    if (st != LOCKS_OK || e != hipSuccess) {
        (void)hipStreamDestroy(s);
        if (g) (void)hipGraphDestroy(g);
        return st != LOCKS_OK ? st : hip_fail(e);
    }
    hipGraphExec_t exec;
    e = hipGraphInstantiate(&exec, g, nullptr, nullptr, 0);
    (void)hipGraphDestroy(g);
    // Upload the executable graph now, so that its first launch costs what
    // every later one does.
    if (e == hipSuccess) {
        e = hipGraphUpload(exec, s);
        if (e == hipSuccess) e = hipStreamSynchronize(s);
        if (e != hipSuccess) (void)hipGraphExecDestroy(exec);
    }
    (void)hipStreamDestroy(s);
    if (e != hipSuccess) return hip_fail(e);
    locks_step_graph* h = new (std::nothrow) locks_step_graph{exec};
    if (!h) {
        (void)hipGraphExecDestroy(exec);
        return LOCKS_ERR_INVALID_ARG;
    }
    *graph = h;
    return LOCKS_OK;
}

locks_status locks_step_graph_launch(locks_step_graph* graph, void* stream) {
    if (!graph) return LOCKS_ERR_INVALID_ARG;
    const hipError_t e = hipGraphLaunch(graph->exec, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? LOCKS_OK : hip_fail(e);
}

void locks_step_graph_destroy(locks_step_graph* graph) {
    if (!graph) return;
    (void)hipGraphExecDestroy(graph->exec);
    delete graph;
}

locks_status locks_probe_stream_read(const void* buf, size_t bytes, float* sink,
                                     int32_t sink_floats, void* stream) {
    if (!buf || !sink || bytes == 0 || bytes % 16 != 0 || sink_floats < 4 ||
        sink_floats % 4 != 0 || sink_floats / 4 > 65536)
        return LOCKS_ERR_INVALID_ARG;
    const hipError_t e = locks::launch_probe_stream(buf, bytes, sink, sink_floats / 4,
                                                    static_cast<hipStream_t>(stream));
    return e == hipSuccess ? LOCKS_OK : hip_fail(e);
}

locks_status locks_probe_summary_read(const float* q, int32_t num_q_heads,
                                      const locks_summaries* summaries,
                                      const locks_page_table* pages, float* page_out,
                                      void* stream) {
    locks_status st = check_summaries(summaries, true);
    if (st != LOCKS_OK) return st;
    if ((st = check_page_table(pages)) != LOCKS_OK) return st;
    if (!q || !page_out || !head_dims_ok(num_q_heads, summaries->num_kv_heads))
        return LOCKS_ERR_INVALID_ARG;
    if (summaries->dtype != LOCKS_F32 ||
        !locks::probe_scan_supported(summaries->page_size, summaries->head_dim, summaries->rank))
        return LOCKS_ERR_UNSUPPORTED;
    locks::ProbeScanParams p{};
    p.q = q;
    p.mu = summaries->mu;
    p.basis = summaries->basis;
    p.coef = summaries->coef;
    p.block_table = pages->block_table;
    p.seq_lens = pages->seq_lens;
    p.batch = pages->batch;
    p.num_q_heads = num_q_heads;
    p.num_kv_heads = summaries->num_kv_heads;
    p.max_pages = pages->max_pages;
    p.num_blocks = summaries->num_blocks;
    p.page_out = page_out;
    const hipError_t e = locks::launch_probe_scan(p, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? LOCKS_OK : hip_fail(e);
}

const char* locks_status_string(int32_t status) {
    switch (status) {
        case LOCKS_OK:
            return "ok";
        case LOCKS_ERR_INVALID_ARG:
            return "invalid argument";
        case LOCKS_ERR_UNSUPPORTED:
            return "unsupported shape or dtype";
        case LOCKS_ERR_WORKSPACE:
            return "workspace missing or too small";
        case LOCKS_ERR_HIP:
            return "HIP error";
        default:
            return "unknown status";
    }
}

int32_t locks_last_hip_error(void) { return g_last_hip_error; }

int32_t locks_version(void) { return 106; }

}  // extern "C"
