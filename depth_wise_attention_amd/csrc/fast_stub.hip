// Placeholder: no specialised kernels yet; every shape takes the general path.
#include "launch.hpp"

namespace attnres {
bool phase1_fast_ok(const Phase1Args&) { return false; }
bool phase2_fast_ok(const Phase2Args&) { return false; }
bool bwd_fast_ok(const BwdArgs&) { return false; }
bool full_fast_ok(const FullArgs&) { return false; }
hipError_t launch_phase1_fast(const Phase1Args&, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_phase2_fast(const Phase2Args&, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_bwd_fast(const BwdArgs&, int64_t*, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_full_fast(const FullArgs&, hipStream_t) { return hipErrorNotSupported; }
}  // namespace attnres
