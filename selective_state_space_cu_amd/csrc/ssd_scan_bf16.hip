// bf16 instances of the fused chunk-walk scan.
#include "ssd_scan.hpp"

namespace ssd {

hipError_t launch_scan_bf16(const ScanArgs &a, int waves, int dstate, hipStream_t stream) {
    switch (dstate) {
    case 16: return launch_scan_waves<uint16_t, 16>(a, waves, stream);
    case 32: return launch_scan_waves<uint16_t, 32>(a, waves, stream);
    case 64: return launch_scan_waves<uint16_t, 64>(a, waves, stream);
    case 128: return launch_scan_waves<uint16_t, 128>(a, waves, stream);
    case 256: return launch_scan_waves<uint16_t, 256>(a, waves, stream);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace ssd
