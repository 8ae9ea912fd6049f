// Stand-ins for the kernel launchers, for a host-only build of the C ABI
// layer (gdr_api.hip, gdr_timing.hip) under AddressSanitizer and
// UndefinedBehaviorSanitizer.  The validation tests never reach a launch;
// if one did, it would report a HIP error instead of touching a device.
#include "gdr_internal.h"

namespace gdr {
hipError_t prefill_launch(const PrefillArgs&, const PrefillLayout&, int, hipStream_t) {
    return hipErrorNotSupported;
}
hipError_t decode_launch(const DecodeArgs&, int, int, hipStream_t) { return hipErrorNotSupported; }
}  // namespace gdr
