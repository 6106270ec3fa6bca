// Placeholder: no specialised kernels yet; every shape takes the general path.
#include "launch.hpp"

namespace attnres {


bool bwd_fast_ok(const BwdArgs&) { return false; }
bool full_fast_ok(const FullArgs&) { return false; }


hipError_t launch_bwd_fast(const BwdArgs&, int64_t*, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_full_fast(const FullArgs&, hipStream_t) { return hipErrorNotSupported; }
}  // namespace attnres
