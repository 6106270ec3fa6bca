// Block AttnRes Phase 1 and backward kernels for blocks that read 11 reps
// (see p1_kernel.hpp and bwd_kernel.hpp).
#include "bwd_kernel.hpp"
#include "p1_kernel.hpp"

namespace attnres {
template <>
hipError_t p1_launch_n<11>(const Phase1Args& a, const P1Plan& p, hipStream_t st) {
  return p1_launch_for<11>(a, p, st);
}
template <>
hipError_t bwd_launch_n<11>(const BwdArgs& a, const BwdPlan& p, int po, bool dry, int64_t* slots_used,
                          hipStream_t st) {
  return bwd_launch_for<11>(a, p, po, dry, slots_used, st);
}
}  // namespace attnres
