// float32 instances of the fused chunk-walk scan.
#include "ssd_scan.hpp"

namespace ssd {

hipError_t launch_scan_f32(const ScanArgs &a, int waves, int dstate, hipStream_t stream) {
    switch (dstate) {
    case 16: return launch_scan_waves<float, 16>(a, waves, stream);
    case 32: return launch_scan_waves<float, 32>(a, waves, stream);
    case 64: return launch_scan_waves<float, 64>(a, waves, stream);
    case 128: return launch_scan_waves<float, 128>(a, waves, stream);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace ssd
