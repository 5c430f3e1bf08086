// Summary scan: dispatch on the stored summary type.  The kernel (per-page
// estimated attention mass from the resident summary alone, aggregated over
// each GQA group; gist.science technical summary, section 2, Reconstructie
// en Selectie and Group-Shared Selection) is in scan_kernel.hpp, compiled
// once per type by scan_f32.hip, scan_bf16.hip and scan_q8q4.hip.
#include "launchers.hpp"

namespace locks {

hipError_t launch_scan_f32(const ScanParams& p, hipStream_t s);
hipError_t launch_scan_bf16(const ScanParams& p, hipStream_t s);
hipError_t launch_scan_q8q4(const ScanParams& p, hipStream_t s);

bool scan_supported(int page_size, int head_dim, int rank) {
    return (page_size == 16 || page_size == 64) && (head_dim == 64 || head_dim == 128) &&
           rank >= 1 && rank <= 16 && rank <= page_size && rank <= head_dim;
}

hipError_t launch_scan(const ScanParams& p, hipStream_t s) {
    if (p.summ_dtype == kSummQ8Q4) return launch_scan_q8q4(p, s);
    if (p.summ_dtype == kSummBF16) return launch_scan_bf16(p, s);
    return launch_scan_f32(p, s);
}

}  // namespace locks
