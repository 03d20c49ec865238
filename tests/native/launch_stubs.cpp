// Launcher stubs for the host-only sanitizer build of the C ABI (api.cpp,
// plan.cpp, schedule.cpp under -fsanitize=address,undefined). That build
// runs only validation, planning and the no-device error paths, which never
// reach a kernel launch; each stub reports hipErrorNotSupported if called.
#include <hip/hip_runtime_api.h>

#include "../../muon_newton_schulz_04_amd/csrc/launch.hpp"

namespace muon {

hipError_t launch_momentum(const LaunchCtx&, const float*, float*, float, int, int) { return hipErrorNotSupported; }
hipError_t launch_apply(const LaunchCtx&, const void*, const float*, float*, float, float) { return hipErrorNotSupported; }
hipError_t launch_normuon(const LaunchCtx&, float, float) { return hipErrorNotSupported; }
hipError_t launch_reset(const LaunchCtx&, float*) { return hipErrorNotSupported; }
hipError_t launch_ns_stage(const LaunchCtx&, const GemmList&, int, const void*, const void*, void*, float, float, float,
                           int, float, int) {
    return hipErrorNotSupported;
}
hipError_t launch_ns_stage_big(const LaunchCtx&, const GemmList&, int, const void*, const void*, void*, float, float,
                               float, int, float, int) {
    return hipErrorNotSupported;
}
hipError_t launch_ns_panel(const LaunchCtx&, const int32_t*, int, const NsCoeffs&, int) { return hipSuccess; }
hipError_t launch_ns_small(const LaunchCtx&, const int32_t*, int, int, const NsCoeffs&, void*, int) {
    return hipErrorNotSupported;
}
size_t ns_small_lds_bytes(int n_pad_max) { return (size_t)n_pad_max; }
hipError_t prepare_ns_small(int) { return hipErrorNotSupported; }
hipError_t static_scratch_address(int, void**) { return hipErrorNotSupported; }

}  // namespace muon
