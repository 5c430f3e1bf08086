// Summary scan: dispatch on the stored summary type.  The kernel (per-page
// estimated attention mass from the resident summary alone, aggregated over
// each GQA group; gist.science technical summary, section 2, Reconstructie
// en Selectie and Group-Shared Selection) is in scan_kernel.hpp, compiled
// once per type by scan_f32.hip, scan_bf16.hip and scan_q8q4.hip.
#include <atomic>

#include "launchers.hpp"

namespace locks {

hipError_t launch_scan_f32(const ScanParams& p, hipStream_t s);
hipError_t launch_scan_bf16(const ScanParams& p, hipStream_t s);
hipError_t launch_scan_q8q4(const ScanParams& p, hipStream_t s);

bool scan_supported(int page_size, int head_dim, int rank) {
    return (page_size == 16 || page_size == 64) && (head_dim == 64 || head_dim == 128) &&
           rank >= 1 && rank <= 16 && rank <= page_size && rank <= head_dim;
}

// Compute units of the current device (0 if the query fails), cached per
// device: a property query, no stream work, so it is safe under capture.
// Threads that race on the first query store the same value.
static int device_compute_units() {
    static std::atomic<int> cached[64];  // 0: not queried yet, -1: the query failed
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
    int n = cached[dev].load(std::memory_order_relaxed);
    if (n == 0) {
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            n <= 0)
            n = -1;
        cached[dev].store(n, std::memory_order_relaxed);
    }
    return n > 0 ? n : 0;
}

hipError_t launch_scan(const ScanParams& p, hipStream_t s) {
    ScanParams q = p;
    q.one_round = 0;
    if (p.summ_dtype == kSummQ8Q4) {
        // the code kernel keeps three waves per SIMD, four SIMDs per CU
        const long waves = (long)p.batch * p.num_kv_heads * ((p.max_pages + kRunPages - 1) / kRunPages);
        q.one_round = waves <= 12L * device_compute_units() ? 1 : 0;
        return launch_scan_q8q4(q, s);
    }
    if (p.summ_dtype == kSummBF16) return launch_scan_bf16(q, s);
    return launch_scan_f32(q, s);
}

}  // namespace locks
