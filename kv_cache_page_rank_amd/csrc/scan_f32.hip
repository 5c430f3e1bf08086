// Summary scan instantiated for fp32 summaries (kernel in scan_kernel.hpp).
#include "scan_kernel.hpp"

namespace locks {

hipError_t launch_scan_f32(const ScanParams& p, hipStream_t s) {
    return launch_scan_of<float>(p, s);
}

}  // namespace locks
