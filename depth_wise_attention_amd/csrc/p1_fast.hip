// Planning and dispatch of the specialised Block AttnRes Phase 1 kernel
// (p1_kernel.hpp).  Every function here is host logic: which kernel variant
// a call runs follows from its sizes and pointer alignment alone, so it can
// be queried (and tested) without a GPU.
#include <stdio.h>

#include "p1_kernel.hpp"

namespace attnres {
namespace {

constexpr int kP1MaxN = 12;
constexpr int kP1MaxS = 8;
// The largest workgroup a variant runs with, and the LDS of one compute unit.
constexpr int kP1MaxB = 512;
constexpr size_t kLdsPerCu = 160 * 1024;

bool p1_aligned16(const void* p) { return p == nullptr || ((uintptr_t)p & 15u) == 0; }

// Length of one wave's reduction row (floats): the dot products and sums of
// squares of a token, padded to a multiple of 8.
int64_t p1_row_floats(int64_t N, int64_t S, int ch, bool mh) { return (((mh ? ch : 1) * S * N + N) + 7) / 8 * 8; }

// The plan of a call, or ch == 0 when the call needs the general kernel.
// Two chunks of 8 channels per thread (the layout the d = 4096, N = 8, S = 4
// block was tuned with) when the N rep rows and S N + N partial sums fit the
// registers twice over: N <= 8 and S <= 4, d a multiple of 1024.  Otherwise
// one chunk per thread, B = d / 8 threads; above d = 4096 that would take
// more than 512 threads, so those shapes run on the general kernel.
P1Plan p1_plan(const Phase1Args& a) {
  P1Plan p;
  if (a.dtype != kBF16 || a.T < 1 || a.T >= ((int64_t)1 << 31)) return p;
  if (a.N < 1 || a.N > kP1MaxN || a.S < 1 || a.S > kP1MaxS) return p;
  if (a.S > 1 && a.orest_dtype != kF16 && a.orest_dtype != kF32) return p;
  if (a.d < 512 || a.d % 512 != 0 || a.H < 1 || a.d % a.H != 0 || (a.d / a.H) % 512 != 0) return p;
  if (!p1_aligned16(a.reps) || !p1_aligned16(a.o0) || !p1_aligned16(a.orest) || !p1_aligned16(a.w) ||
      !p1_aligned16(a.gain))
    return p;
  const bool mh = a.H > 1;
  const int ch = (a.N <= 8 && a.S <= 4 && a.d % 1024 == 0) ? 2 : 1;
  const int64_t B = a.d / (8 * ch);
  if (B % 64 != 0 || B < 64 || B > kP1MaxB) return p;
  const size_t q_bytes = (size_t)(a.S * a.d * 4);
  const size_t red_bytes = (size_t)(2 * (B / 64) * p1_row_floats(a.N, a.S, ch, mh) * 4);
  if (q_bytes + red_bytes > kLdsPerCu) return p;
  p.ch = ch;
  p.mh = mh;
  p.B = (int)B;
  p.lds = q_bytes + red_bytes;
  return p;
}

}  // namespace

bool phase1_fast_ok(const Phase1Args& a) { return p1_plan(a).ch != 0; }

void phase1_fast_variant(const Phase1Args& a, char* buf, size_t len) {
  const P1Plan p = p1_plan(a);
  if (len == 0) return;
  if (p.ch == 0) {
    buf[0] = '\0';
    return;
  }
  snprintf(buf, len, "phase1_fast<N=%lld,S=%lld,CH=%d,MH=%d> B=%d lds=%zu", (long long)a.N, (long long)a.S, p.ch,
           p.mh ? 1 : 0, p.B, p.lds);
}

hipError_t launch_phase1_fast(const Phase1Args& a, hipStream_t st) {
  const P1Plan p = p1_plan(a);
  if (p.ch == 0) return hipErrorNotSupported;
  switch (a.N) {
    case 1: return p1_launch_n<1>(a, p, st);
    case 2: return p1_launch_n<2>(a, p, st);
    case 3: return p1_launch_n<3>(a, p, st);
    case 4: return p1_launch_n<4>(a, p, st);
    case 5: return p1_launch_n<5>(a, p, st);
    case 6: return p1_launch_n<6>(a, p, st);
    case 7: return p1_launch_n<7>(a, p, st);
    case 8: return p1_launch_n<8>(a, p, st);
    case 9: return p1_launch_n<9>(a, p, st);
    case 10: return p1_launch_n<10>(a, p, st);
    case 11: return p1_launch_n<11>(a, p, st);
    default: return p1_launch_n<12>(a, p, st);
  }
}

}  // namespace attnres
