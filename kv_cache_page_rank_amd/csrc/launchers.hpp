// Host-side launchers of the gfx950 kernels (defined next to each kernel).
// Each returns the hipError_t of its launch.  Shapes are validated by the
// C-ABI layer before any launcher is called.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace locks {

// Pages per run: the scan may also write, per (b, g), the maximum page mass
// of every run of kRunPages consecutive pages; the top-k uses these maxima
// to read only the runs that can hold a winner.
constexpr int kRunPages = 16;

// Stored summary element types.
enum SummDtype : int32_t { kSummF32 = 0, kSummBF16 = 1, kSummQ8Q4 = 2 };

struct ScanParams {
    const float* q;        // [B][Hq][D]
    const void* mu;        // [NB][Hkv][D]       fp32, bf16 or int8 codes (summ_dtype)
    const void* basis;     // [NB][Hkv][r][D]    (int4 codes: [NB][Hkv][r][D/2] bytes)
    const void* coef;      // [NB][Hkv][P][r]
    const float* scales;   // kSummQ8Q4: [NB][Hkv][1 + 2r]
    int32_t summ_dtype;
    const int32_t* block_table;
    const int32_t* seq_lens;
    const int32_t* summarized;  // [B] or null: leading pages with summaries (candidates)
    int32_t batch, num_q_heads, num_kv_heads, max_pages, num_blocks;
    int32_t page_size, head_dim, rank;
    float* page_logmass;   // [B][Hkv][max_pages]
    float* head_logmass;   // [B][Hq][max_pages] or null
    float* run_max;        // [B][Hkv][ceil(max_pages / kRunPages)] or null
    int32_t one_round;     // set by launch_scan: every wave of the launch is resident at once
};
hipError_t launch_scan(const ScanParams& p, hipStream_t s);
bool scan_supported(int page_size, int head_dim, int rank);

// Mean-of-share group scores from per-head estimates.
struct ShareParams {
    const float* head_logmass;  // [B][Hq][max_pages]
    const int32_t* seq_lens;
    const int32_t* summarized;  // [B] or null: leading pages with summaries (candidates)
    int32_t batch, num_q_heads, num_kv_heads, max_pages, page_size;
    float* head_total;          // [B][Hq] workspace
    float* page_logmass;        // [B][Hkv][max_pages]
    float* run_max;             // [B][Hkv][ceil(max_pages / kRunPages)] or null
};
hipError_t launch_share(const ShareParams& p, hipStream_t s);

struct TopkParams {
    const float* page_logmass;  // [B][Hkv][max_pages]
    const int32_t* seq_lens;
    const int32_t* summarized;  // [B] or null: leading pages with summaries (candidates)
    int32_t batch, num_kv_heads, max_pages, page_size, k_req, width;
    int32_t* sel_pages;         // [B][Hkv][width]
    float* sel_logmass;         // [B][Hkv][width] or null
    const float* run_max;       // [B][Hkv][ceil(max_pages / kRunPages)] or null
};
constexpr int kTopkMaxPages = 32768;
hipError_t launch_topk(const TopkParams& p, hipStream_t s);

struct AttnParams {
    const float* q;            // [B][Hq][D]
    const void* k;             // [NB][Hkv][P][D]
    const void* v;             // [NB][Hkv][D][P]
    int32_t bf16;              // cache dtype
    const int32_t* block_table;
    const int32_t* seq_lens;
    const int32_t* summarized;  // [B] or null: leading pages with summaries (candidates)
    const int32_t* sel_pages;  // [B][Hkv][k_sel] (sparse) or null (dense)
    int32_t batch, num_q_heads, num_kv_heads, max_pages, num_blocks;
    int32_t page_size, head_dim;
    int32_t k_sel;             // sparse: selected slots per (b, g)
    int32_t pages_per_split;   // dense: pages per split
    int32_t num_splits;        // sparse: k_sel + 1 (last = partial page); dense: ceil(max_pages / pps)
    int32_t num_parts;         // partials per (b, h) after the in-workgroup combine (set by the launcher)
    float* part_ml;            // [B][Hq][num_parts][2] (max, sum) in log2 units, num_parts <= num_splits
    float* part_o;             // [B][Hq][num_parts][D] unnormalised outputs
    void* out;                 // [B][Hq][D] cache dtype
    float* out_lse;            // [B][Hq] or null
};
hipError_t launch_attend(const AttnParams& p, hipStream_t s);
bool attend_supported(int bf16, int page_size, int head_dim);
int dense_pages_per_split(int batch, int num_kv_heads, int max_pages);

struct BuildParams {
    const void* k;             // [NB][Hkv][P][D]
    int32_t bf16;
    const int32_t* block_table;
    const int32_t* seq_lens;
    const int32_t* page_begin; // [B] or null
    int32_t refresh_pages;     // > 0: only pages page_begin[b] .. + refresh_pages - 1
    int32_t batch, num_kv_heads, max_pages, num_blocks;
    int32_t page_size, head_dim, rank;
    void* mu;              // fp32, bf16 or int8/int4 codes (out_dtype)
    void* basis;
    void* coef;
    float* scales;         // kSummQ8Q4: [NB][Hkv][1 + 2r]
    int32_t out_dtype;     // SummDtype
};
hipError_t launch_build(const BuildParams& p, hipStream_t s);
// After a refresh of pages [page_begin[b], min(page_begin[b] + max_new_pages,
// full pages)): summarized[b] advances to the end of that range when it
// reached at least page_begin[b] (no gap).  One thread per sequence.
hipError_t launch_advance_summarized(const int32_t* seq_lens, const int32_t* page_begin,
                                     int32_t* summarized, int32_t batch, int32_t page_size,
                                     int32_t max_pages, int32_t max_new_pages, hipStream_t s);
bool build_supported(int page_size, int head_dim, int rank);

// Shared-basis sketch (ablation baseline): the centroid of every full page
// and its tokens' coordinates in one basis per KV head, written as fp32
// summaries with that basis copied to every block.  Uses BuildParams (mu,
// basis, coef: fp32 outputs) and shared_basis [Hkv][rank][D].
hipError_t launch_sketch(const BuildParams& p, const float* shared_basis, hipStream_t s);

// fp32 summaries -> int8 / int4 codes and scales, every unit of the pools.
struct QuantParams {
    const float* mu;       // [units][D]
    const float* basis;    // [units][r][D]
    const float* coef;     // [units][P][r]
    int8_t* mu_q;          // [units][D]
    uint8_t* basis_q;      // [units][r][D/2]
    int8_t* coef_q;        // [units][P][r]
    float* scales;         // [units][1 + 2r]
    int64_t units;
    int32_t page_size, head_dim, rank;
};
hipError_t launch_quantize(const QuantParams& p, hipStream_t s);

// Measurement probes (not part of the decode step): a streaming read, and a
// read of the fp32 summary scan's bytes in the scan's access pattern.
struct ProbeScanParams {
    const float* q;            // [B][Hq][D]
    const void* mu;            // fp32 summaries, as ScanParams
    const void* basis;
    const void* coef;
    const int32_t* block_table;
    const int32_t* seq_lens;
    int32_t batch, num_q_heads, num_kv_heads, max_pages, num_blocks;
    float* page_out;           // [B][Hkv][max_pages], one value per page
};
hipError_t launch_probe_stream(const void* buf, size_t bytes, float* sink, int32_t blocks,
                               hipStream_t s);
hipError_t launch_probe_scan(const ProbeScanParams& p, hipStream_t s);
bool probe_scan_supported(int page_size, int head_dim, int rank);

}  // namespace locks
