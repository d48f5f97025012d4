// Stand-ins for the kernel launchers, linked only into the sanitizer build of
// the host layer (tests/test_sanitizers.py).  That build runs without a GPU, so
// every call stops at the device check before any launcher is reached; each
// stand-in reports failure should one be called anyway.
#include "gdn_internal.h"

namespace gdn {
hipError_t launch_decode(const DecodeParams &, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_fused_scan(const ScanParams &, bool, int, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_piped_scan(const ScanParams &, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_plan(const void *, int, int, int64_t, SegEntry *, int32_t *, int32_t *, int, hipStream_t) {
    return hipErrorNotSupported;
}
hipError_t launch_fixup(const FixParams &, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_prep(const ScanParams &, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_prepared_scan(const ScanParams &, int, hipStream_t) { return hipErrorNotSupported; }
}  // namespace gdn
