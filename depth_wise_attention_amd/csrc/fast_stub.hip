// The Full AttnRes forward has no specialised kernel yet; every shape takes
// the general path.
#include "launch.hpp"

namespace attnres {
bool full_fast_ok(const FullArgs&) { return false; }
hipError_t launch_full_fast(const FullArgs&, hipStream_t) { return hipErrorNotSupported; }
}  // namespace attnres
