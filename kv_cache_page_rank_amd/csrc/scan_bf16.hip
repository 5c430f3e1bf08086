// Summary scan instantiated for bf16 summaries (kernel in scan_kernel.hpp).
#include "scan_kernel.hpp"

namespace locks {

hipError_t launch_scan_bf16(const ScanParams& p, hipStream_t s) {
    return launch_scan_of<uint16_t>(p, s);
}

}  // namespace locks
