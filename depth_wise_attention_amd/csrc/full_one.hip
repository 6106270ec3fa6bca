// Full AttnRes forward for one destination over up to 64 sources (gfx950,
// bf16 I/O): the call a model makes per sublayer, at any depth up to 63
// sublayers (b-lab.team summary §1; dimensionstp "Attention Residuals Review"
// §3 (2) runs 54).  With H heads (chatpaper MHAR abstract) each head is a run
// of whole 512-channel waves with its own dot products and softmax; the RMS
// is over the whole d.  With one query the contractions per token are two
// vectors of n_src dot products over d, far too small for the matrix cores;
// what matters is reading each source row once.
//
// One workgroup of d / 8 threads owns one token at a time; thread tid owns
// channels 8 tid .. 8 tid + 7.  The sources are taken in NT = 1 or 2 tiles of
// 32 rows, each held in registers (16-byte buffer loads, one register per
// row; a row past n_src is loaded with a zero-record descriptor, which reads
// nothing and gives zeros):
//   1. per row, the sum of squares and q . v over the thread's channels;
//   2. transposing reductions over the wave (16 rows at a time) and a sum
//      over the waves through LDS (one barrier per tile);
//   3. the tile's scores, and the depth softmax carried across the tiles
//      online: with m the running maximum and l the running sum of
//      exp(s - m), a tile with maximum m' rescales the running sum and the
//      weighted sum by exp(m - max(m, m'));
//   4. the weighted sum sum_i exp(s_i - m) v_i from the registers; as each row
//      is used for the last time its register takes the next tile's row (or
//      the next token's first tile), so the loads overlap the rest of the work.
// The output is the weighted sum over the running sum, rounded once to bf16.
#include <math.h>

#include "common.hpp"
#include "launch.hpp"
#include "xlane.hpp"

namespace attnres {
namespace {

constexpr int kOTile = 32;   // source rows per register tile
constexpr int kOMaxW = 8;    // waves per workgroup at most (d <= 4096)

template <int NT>
__global__ __launch_bounds__(512, 2) void k_full_one(FullArgs a) {
  __shared__ float red[2][kOMaxW][2 * kOTile];  // per buffer and wave: 32 sums of squares, then 32 dot products
  const int tid = threadIdx.x, lane = lane_id();
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int W = (int)blockDim.x >> 6;
  const int wph = W / a.H, hw0 = wave / wph * wph;  // waves per head; this head's first wave
  const int d = (int)a.d, n_src = (int)a.n_src;
  const int64_t T = a.T, plane = T * d;
  const bf16_t* src = static_cast<const bf16_t*>(a.src);
  bf16_t* out = static_cast<bf16_t*>(a.out);
  const uint32_t coff = (uint32_t)tid * 16u;  // this thread's byte offset in a row
  const float inv_d = 1.0f / (float)d;

  float q[8];  // q = w * g of the destination, for this thread's channels
  if (a.gain != nullptr)
    fold_q8<true>(a.w + 8 * tid, a.gain + 8 * tid, q);
  else
    fold_q8<false>(a.w + 8 * tid, nullptr, q);

  // Row r of token t (the address of a row past n_src is the last real row's,
  // which its zero-record load never reads), from opaque scalar copies of the plane size and
  // the source count taken per tile: the 64 row offsets are loop-invariant,
  // and held across the token loop they would take more scalar registers
  // than there are.
  auto row = [&](int64_t pl, int ns, int64_t t, int r) { return src + (int64_t)(r < ns ? r : ns - 1) * pl + t * d; };
  uint4 v[kOTile];
  int64_t t = blockIdx.x;
  if (t < T) {
#pragma unroll
    for (int k = 0; k < kOTile; ++k) v[k] = ld16_rec(row(plane, n_src, t, k), coff, k < n_src ? 0x7fffffff : 0);
  }
  // One flat loop over (token, tile) pairs, so that the row registers take
  // the same physical registers in every iteration.
  int buf = 0;
  float m = -INFINITY, lsum = 0.f, acc[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) acc[k] = 0.f;
  int tl = 0;
#pragma unroll 1
  while (t < T) {
    // The rows that refill the registers: this token's next tile, or the
    // next token's first.
    const bool last = tl == NT - 1;
    const int64_t tn = last ? t + gridDim.x : t;
    const int rn0 = last ? 0 : (tl + 1) * kOTile;
    const bool more = tn < T;
    const int64_t tr = more ? tn : t;       // a real token for the row addresses
    int64_t pl = plane;
    int ns = n_src;
    asm volatile("" : "+s"(pl), "+s"(ns));

    // 1-2. sums of squares and dot products over this thread's channels,
    // reduced over the wave for 16 rows at a time (32 values: lane L ends
    // with value L >> 1), which keeps the partials to 32 registers.
    int rl = lane;
    asm volatile("" : "+v"(rl));
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      float part[kOTile];  // sums of squares of rows 16 h .. 16 h + 15, then their dot products
#pragma unroll
      for (int k = 0; k < 16; ++k) {
        float x[8];
        unpack_bf8(v[16 * h + k], x);
        float ss = 0.f, dt = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          ss = fmaf(x[e], x[e], ss);
          dt = fmaf(q[e], x[e], dt);
        }
        part[k] = ss;
        part[16 + k] = dt;
      }
      const float tot = transpose_reduce_pow2<kOTile>(part);
      const int pv = rl >> 1;
      if ((rl & 1) == 0) red[buf][wave][pv < 16 ? 16 * h + pv : kOTile + 16 * h + (pv - 16)] = tot;
    }
    lds_barrier();
    const int li = rl & (kOTile - 1);  // both half-waves take rows 0..31: every lane holds the same totals
    // The sum of squares is over every wave (the whole d), the dot product
    // over the waves of this wave's head (H heads of W / H whole waves).
    float ss = 0.f, dt = 0.f;
    for (int w2 = 0; w2 < W; ++w2) ss += red[buf][w2][li];
    for (int w2 = hw0; w2 < hw0 + wph; ++w2) dt += red[buf][w2][kOTile + li];
    // 3. scores and the online depth softmax
    const bool valid = tl * kOTile + li < n_src;
    const float s = valid ? dt / sqrtf(ss * inv_d + a.eps) : -INFINITY;
    const float m_new = fmaxf(m, group_max<kOTile>(s));
    const float scale = expf(m - m_new);  // 0 for the first tile (m = -inf)
    const float e = valid ? expf(s - m_new) : 0.f;
    lsum = lsum * scale + group_sum<kOTile>(e);
    m = m_new;
#pragma unroll
    for (int k = 0; k < 8; ++k) acc[k] *= scale;
    // 4. the weighted sum, refilling each row after its last use
#pragma unroll
    for (int k = 0; k < kOTile; ++k) {
      // Unpack the row again: the fp32 copy from step 1 would need 256
      // registers across the barrier.
      uint4 u = v[k];
      asm volatile("" : "+v"(u.x), "+v"(u.y), "+v"(u.z), "+v"(u.w));
      float x[8];
      unpack_bf8(u, x);
      // Past the last token, and for rows past n_src, the load reads nothing.
      v[k] = ld16_rec(row(pl, ns, tr, rn0 + k), coff, more && rn0 + k < ns ? 0x7fffffff : 0);
      const float al = read_lane(e, k);
#pragma unroll
      for (int c = 0; c < 8; ++c) acc[c] = fmaf(al, x[c], acc[c]);
      __builtin_amdgcn_sched_barrier(0);  // one row's floats at a time
    }
    buf ^= 1;
    if (last) {
      const float inv = 1.0f / lsum;
      const uint4 o = make_uint4(pack_bf2(acc[0] * inv, acc[1] * inv), pack_bf2(acc[2] * inv, acc[3] * inv),
                                 pack_bf2(acc[4] * inv, acc[5] * inv), pack_bf2(acc[6] * inv, acc[7] * inv));
      st16_rec(out + t * d, coff, 0x7fffffff, o);
      m = -INFINITY;
      lsum = 0.f;
#pragma unroll
      for (int k = 0; k < 8; ++k) acc[k] = 0.f;
      tl = 0;
      t = tn;
    } else {
      ++tl;
    }
  }
}

}  // namespace

bool full_one_ok(const FullArgs& a) {
  auto al16 = [](const void* p) { return p == nullptr || ((uintptr_t)p & 15u) == 0; };
  // Heads of whole 512-channel waves: H = 1, 2, 4 or 8 with d / H a multiple of 512.
  const bool heads = (a.H == 1 || a.H == 2 || a.H == 4 || a.H == 8) && (a.d / a.H) % 512 == 0;
  return a.dtype == kBF16 && heads && a.n_dst == 1 && a.n_src >= 1 && a.n_src <= 2 * kOTile && a.T >= 1 &&
         a.d >= 512 && a.d % 512 == 0 && a.d <= 8 * 64 * kOMaxW && al16(a.src) && al16(a.out) && al16(a.w) &&
         al16(a.gain);
}

namespace {
template <int NT>
hipError_t launch_one(const FullArgs& a, hipStream_t st) {
  const int B = (int)(a.d / 8);
  int per_cu = 0;
  const hipError_t e = blocks_per_cu(reinterpret_cast<const void*>(k_full_one<NT>), B, &per_cu);
  if (e != hipSuccess) return e;
  int64_t grid = (int64_t)num_cus() * (per_cu < 1 ? 1 : per_cu);
  if (grid > a.T) grid = a.T;
  hipLaunchKernelGGL(k_full_one<NT>, dim3((unsigned)grid), dim3((unsigned)B), 0, st, a);
  return hipGetLastError();
}
}  // namespace

hipError_t launch_full_one(const FullArgs& a, hipStream_t st) {
  return a.n_src > kOTile ? launch_one<2>(a, st) : launch_one<1>(a, st);
}

}  // namespace attnres
