// Planning and dispatch of the specialised Block AttnRes backward
// (bwd_kernel.hpp).  Host logic only: the variant a call runs follows from its
// sizes and pointer alignment, so it can be queried without a GPU.
#include <stdio.h>

#include "bwd_kernel.hpp"

namespace attnres {
namespace {

constexpr int kBwdMaxN = 12;
constexpr int kBwdMaxS = 8;    // more than kBwdChunk destinations run as two chunks
constexpr int kBwdChunk = kBwdChunkMax;
constexpr size_t kBwdLdsPerCu = 160 * 1024;

bool bwd_aligned16(const void* p) { return p == nullptr || ((uintptr_t)p & 15u) == 0; }

// Floats of one wave's reduction row for S destinations reading N reps and
// S - po partials (po as the kernel's PO).
int64_t bwd_row_floats(int64_t N, int64_t S, int po) { return (N * (1 + 2 * S) + (S - po) * 3 + 7) / 8 * 8; }

size_t bwd_lds(int64_t B, int64_t N, int64_t S, int po) {
  return (size_t)(S * B * 32) + (size_t)(2 * (B / 64) * bwd_row_floats(N, S, po) * 4);
}

// A block of S destinations as chunks: [0, s0) with PO = 1, then [s0, S) with
// PO = 0 when S > kBwdChunk (halves, the first the larger).
int64_t bwd_first_chunk(int64_t S) { return S <= kBwdChunk ? S : (S + 1) / 2; }

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
  const int64_t s0 = bwd_first_chunk(a.S);
  size_t lds = bwd_lds(B, a.N, s0, 1);
  if (s0 < a.S) {
    const size_t l1 = bwd_lds(B, a.N, a.S - s0, 0);
    if (l1 > lds) lds = l1;
  }
  if (lds > kBwdLdsPerCu) return p;
  p.B = (int)B;
  p.hh = a.H;
  p.lds = lds;
  p.s0 = (int)s0;
  return p;
}

hipError_t bwd_launch_chunk(const BwdArgs& c, const BwdPlan& p, int po, bool dry, int64_t* slots_used,
                            hipStream_t st) {
  BwdPlan q = p;
  q.lds = bwd_lds(p.B, c.N, c.S, po);
  switch (c.N) {
    case 1: return bwd_launch_n<1>(c, q, po, dry, slots_used, st);
    case 2: return bwd_launch_n<2>(c, q, po, dry, slots_used, st);
    case 3: return bwd_launch_n<3>(c, q, po, dry, slots_used, st);
    case 4: return bwd_launch_n<4>(c, q, po, dry, slots_used, st);
    case 5: return bwd_launch_n<5>(c, q, po, dry, slots_used, st);
    case 6: return bwd_launch_n<6>(c, q, po, dry, slots_used, st);
    case 7: return bwd_launch_n<7>(c, q, po, dry, slots_used, st);
    case 8: return bwd_launch_n<8>(c, q, po, dry, slots_used, st);
    case 9: return bwd_launch_n<9>(c, q, po, dry, slots_used, st);
    case 10: return bwd_launch_n<10>(c, q, po, dry, slots_used, st);
    case 11: return bwd_launch_n<11>(c, q, po, dry, slots_used, st);
    default: return bwd_launch_n<12>(c, q, po, dry, slots_used, st);
  }
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
  snprintf(buf, len, "bwd_fast<N=%lld,S=%lld,HH=%d,S0=%d> B=%d lds=%zu", (long long)a.N, (long long)a.S, p.hh,
           p.s0, p.B, p.lds);
}

// Both chunks of a split block run on one grid (the smaller of the two
// kernels' occupancy grids), so slab b holds every destination's Z row for
// the tokens workgroup b visited, and one reduction over the slabs serves
// the whole block.  The first chunk writes its rep gradients in fp32 to the
// workspace after the slabs; the second reads the partials from b_{s0}, the
// upstream gradients, queries and gains from destination s0 on, adds its rep
// gradients to the first chunk's and rounds once.
hipError_t launch_bwd_fast(const BwdArgs& a, int64_t* slots_used, hipStream_t st) {
  const BwdPlan p = bwd_plan(a);
  if (p.B == 0) return hipErrorNotSupported;
  const int64_t td = a.T * a.d;
  BwdArgs c0 = a;
  c0.S = p.s0;
  c0.zld = a.S * a.d;
  c0.rep_mode = 0;
  if (p.s0 == a.S) return bwd_launch_chunk(c0, p, 1, false, slots_used, st);
  // fp32 rep gradients of the first chunk, after the a.slots Z slabs.
  c0.rep32 = a.zslots + a.slots * a.S * a.d;
  c0.rep_mode = 1;

  BwdArgs c1 = a;
  const int64_t s0 = p.s0;
  c1.S = a.S - s0;
  c1.partials = static_cast<const bf16_t*>(a.partials) + (s0 - 1) * td;
  c1.d_partials = static_cast<bf16_t*>(a.d_partials) + (s0 - 1) * td;
  c1.dh = static_cast<const bf16_t*>(a.dh) + s0 * td;
  c1.w = a.w + s0 * a.d;
  if (a.gain != nullptr) c1.gain = a.gain + s0 * a.gain_ld;
  c1.zslots = a.zslots + s0 * a.d;
  c1.zld = a.S * a.d;
  c1.rep32 = c0.rep32;
  c1.rep_mode = 2;
  int64_t g0 = 0, g1 = 0;
  hipError_t e = bwd_launch_chunk(c0, p, 1, true, &g0, st);
  if (e == hipSuccess) e = bwd_launch_chunk(c1, p, 0, true, &g1, st);
  if (e != hipSuccess) return e;
  const int64_t grid = g0 < g1 ? g0 : g1;
  c0.slots = c1.slots = grid;
  e = bwd_launch_chunk(c0, p, 1, false, &g0, st);
  if (e == hipSuccess) e = bwd_launch_chunk(c1, p, 0, false, &g1, st);
  *slots_used = grid;
  return e;
}

}  // namespace attnres
