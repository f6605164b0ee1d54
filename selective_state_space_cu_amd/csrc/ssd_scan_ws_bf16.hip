// bf16 instance of the warp-specialised scan (dstate 128, 64-column headdim
// tiles, chunk_size >= 64).
#include "ssd_scan_ws.hpp"

namespace ssd {

hipError_t launch_scan_ws_bf16(const ScanArgs &a, int dstate, hipStream_t stream) {
    switch (dstate) {
    case 128: return launch_scan_ws_instance<128>(a, stream);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace ssd
