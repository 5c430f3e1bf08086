// Summary scan instantiated for int8 / int4 code summaries (kernel in scan_kernel.hpp).
#include "scan_kernel.hpp"

namespace locks {

hipError_t launch_scan_q8q4(const ScanParams& p, hipStream_t s) {
    return launch_scan_of<int8_t>(p, s);
}

}  // namespace locks
