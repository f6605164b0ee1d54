// bf16 instance of the split-state scan (dstate 128, 64-column headdim tiles).
#include "ssd_scan_split.hpp"

namespace ssd {

hipError_t launch_scan_split_bf16(const ScanArgs &a, int dstate, hipStream_t stream) {
    switch (dstate) {
    case 128: return launch_scan_split_instance<128>(a, stream);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace ssd
