// Planning and dispatch of the specialised Block AttnRes backward
// (bwd_kernel.hpp).  Host logic only: the variant a call runs follows from its
// sizes and pointer alignment, so it can be queried without a GPU.
#include <stdio.h>

#include "bwd_kernel.hpp"

namespace attnres {
namespace {

constexpr int kBwdMaxN = 12;
constexpr int kBwdMaxS = 4;
constexpr size_t kBwdLdsPerCu = 160 * 1024;

bool bwd_aligned16(const void* p) { return p == nullptr || ((uintptr_t)p & 15u) == 0; }

int64_t bwd_row_floats(int64_t N, int64_t S) { return (N * (1 + 2 * S) + (S - 1) * 3 + 7) / 8 * 8; }

// One chunk of 8 channels per thread (B = d / 8 threads, at most 512):
// d a multiple of 512 up to 4096; heads of whole waves, H in {1, 2, 4, 8}
// dividing the d / 512 waves.
BwdPlan bwd_plan(const BwdArgs& a) {
  BwdPlan p;
  if (a.dtype != kBF16 || a.T < 1 || a.T >= ((int64_t)1 << 31) || a.slots < 1) return p;
  if (a.N < 1 || a.N > kBwdMaxN || a.S < 1 || a.S > kBwdMaxS) return p;
  if (a.d < 512 || a.d > 4096 || a.d % 512 != 0) return p;
  const int64_t waves = a.d / 512;
  if (a.H != 1 && a.H != 2 && a.H != 4 && a.H != 8) return p;
  if (waves % a.H != 0) return p;
  if (!bwd_aligned16(a.reps) || !bwd_aligned16(a.partials) || !bwd_aligned16(a.dh) || !bwd_aligned16(a.d_reps) ||
      !bwd_aligned16(a.d_partials) || !bwd_aligned16(a.zslots) || !bwd_aligned16(a.w) || !bwd_aligned16(a.gain))
    return p;
  const int64_t B = a.d / 8;
  const size_t lds = (size_t)(a.S * B * 32) + (size_t)(2 * (B / 64) * bwd_row_floats(a.N, a.S) * 4);
  if (lds > kBwdLdsPerCu) return p;
  p.B = (int)B;
  p.hh = a.H;
  p.lds = lds;
  return p;
}

}  // namespace

bool bwd_fast_ok(const BwdArgs& a) { return bwd_plan(a).B != 0; }

void bwd_fast_variant(const BwdArgs& a, char* buf, size_t len) {
  const BwdPlan p = bwd_plan(a);
  if (len == 0) return;
  if (p.B == 0) {
    buf[0] = '\0';
    return;
  }
  snprintf(buf, len, "bwd_fast<N=%lld,S=%lld,HH=%d> B=%d lds=%zu", (long long)a.N, (long long)a.S, p.hh, p.B,
           p.lds);
}

hipError_t launch_bwd_fast(const BwdArgs& a, int64_t* slots_used, hipStream_t st) {
  const BwdPlan p = bwd_plan(a);
  if (p.B == 0) return hipErrorNotSupported;
  switch (a.N) {
    case 1: return bwd_launch_n<1>(a, p, slots_used, st);
    case 2: return bwd_launch_n<2>(a, p, slots_used, st);
    case 3: return bwd_launch_n<3>(a, p, slots_used, st);
    case 4: return bwd_launch_n<4>(a, p, slots_used, st);
    case 5: return bwd_launch_n<5>(a, p, slots_used, st);
    case 6: return bwd_launch_n<6>(a, p, slots_used, st);
    case 7: return bwd_launch_n<7>(a, p, slots_used, st);
    case 8: return bwd_launch_n<8>(a, p, slots_used, st);
    case 9: return bwd_launch_n<9>(a, p, slots_used, st);
    case 10: return bwd_launch_n<10>(a, p, slots_used, st);
    case 11: return bwd_launch_n<11>(a, p, slots_used, st);
    default: return bwd_launch_n<12>(a, p, slots_used, st);
  }
}

}  // namespace attnres
