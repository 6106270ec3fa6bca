// Full AttnRes forward for one destination over up to 64 sources (gfx950,
// bf16 I/O): the call a model makes per sublayer, at any depth up to 63
// sublayers (b-lab.team summary §1; dimensionstp "Attention Residuals Review"
// §3 (2) runs 54).  With H heads (chatpaper MHAR abstract) each head is a run
// of whole waves (64 C channels each) with its own dot products and softmax;
// the RMS is over the whole d.  With one query the contractions per token are two
// vectors of n_src dot products over d, far too small for the matrix cores;
// what matters is reading each source row once.
//
// One workgroup of d / C threads owns one token at a time; thread tid owns
// channels C tid .. C tid + C - 1.  The sources are taken in NT register
// tiles of R rows (four registers a row at C = 8, two at C = 4): one 16-row
// tile of 8 channels for up to 16 sources, one 32-row tile of 8
// channels for up to 32 sources, one 64-row tile of 4 channels for 33 .. 64
// with d <= 2048, two 32-row tiles of 8 channels for 33 .. 64 above.  A row
// past n_src is loaded with a zero-record descriptor, which reads nothing and
// gives zeros.  Per tile:
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
#include "row_piece.hpp"
#include "xlane.hpp"

namespace attnres {
namespace {

constexpr int kOMaxW = 8;    // waves per workgroup at most
// 33 .. 64 sources with d <= 2048 and heads of whole 512-channel waves: one
// 64-row tile of 4 channels per thread (true) or two 32-row tiles of 8
// (false).  Measured at 55 sources, T = 4096, d = 2048: 201 us against 192 us,
// so the 64-row tile is kept for heads of 256 channels.
constexpr bool kOneRows64 = false;

template <int NT, int C, int R>
__global__ __launch_bounds__(512, 2) void k_full_one(FullArgs a) {
  // R rows per register tile: R C / 2 registers (128 for the full tiles, 64
  // for the 16-row tile of shallow calls, which leaves room for more tokens
  // in flight per CU).
  typedef typename PieceOf<C>::type P;
  __shared__ float red[2][kOMaxW][2 * R];  // per buffer and wave: R sums of squares, then R dot products
  const int tid = threadIdx.x, lane = lane_id();
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int W = (int)blockDim.x >> 6;
  const int wph = W / a.H, hw0 = wave / wph * wph;  // waves per head; this head's first wave
  const int d = (int)a.d, n_src = (int)a.n_src;
  const int64_t T = a.T, plane = T * d;
  const bf16_t* src = static_cast<const bf16_t*>(a.src);
  bf16_t* out = static_cast<bf16_t*>(a.out);
  const uint32_t coff = (uint32_t)tid * (2u * C);  // this thread's byte offset in a row
  const float inv_d = 1.0f / (float)d;

  float q[C];  // q = w * g of the destination, for this thread's channels
  if (a.gain != nullptr)
    fold_q<C>(a.w + C * tid, a.gain + C * tid, q);
  else
    fold_q<C>(a.w + C * tid, nullptr, q);

  // Row r of token t (the address of a row past n_src is the last real row's,
  // which its zero-record load never reads), from opaque scalar copies of the
  // plane size and the source count taken per tile: the row offsets are
  // loop-invariant, and held across the token loop they would take more
  // scalar registers than there are.
  auto row = [&](int64_t pl, int ns, int64_t t, int r) { return src + (int64_t)(r < ns ? r : ns - 1) * pl + t * d; };
  P v[R];
  int64_t t = blockIdx.x;
  if (t < T) {
#pragma unroll
    for (int k = 0; k < R; ++k) v[k] = piece_ld<C>(row(plane, n_src, t, k), coff, k < n_src ? 0x7fffffff : 0);
  }
  // One flat loop over (token, tile) pairs, so that the row registers take
  // the same physical registers in every iteration.
  int buf = 0;
  float m = -INFINITY, lsum = 0.f, acc[C];
#pragma unroll
  for (int c = 0; c < C; ++c) acc[c] = 0.f;
  int tl = 0;
#pragma unroll 1
  while (t < T) {
    // The rows that refill the registers: this token's next tile, or the
    // next token's first.
    const bool last = tl == NT - 1;
    const int64_t tn = last ? t + gridDim.x : t;
    const int rn0 = last ? 0 : (tl + 1) * R;
    const bool more = tn < T;
    const int64_t tr = more ? tn : t;  // a real token for the row addresses
    int64_t pl = plane;
    int ns = n_src;
    asm volatile("" : "+s"(pl), "+s"(ns));

    // 1-2. sums of squares and dot products over this thread's channels,
    // reduced over the wave for 16 rows at a time (32 values: lane L ends
    // with value L >> 1), which keeps the partials to 32 registers.
    int rl = lane;
    asm volatile("" : "+v"(rl));
#pragma unroll
    for (int h = 0; h < R / 16; ++h) {
      float part[32];  // sums of squares of rows 16 h .. 16 h + 15, then their dot products
#pragma unroll
      for (int k = 0; k < 16; ++k) {
        float x[C];
        piece_unpack(v[16 * h + k], x);
        float ss = 0.f, dt = 0.f;
#pragma unroll
        for (int c = 0; c < C; ++c) {
          ss = fmaf(x[c], x[c], ss);
          dt = fmaf(q[c], x[c], dt);
        }
        part[k] = ss;
        part[16 + k] = dt;
      }
      const float tot = transpose_reduce_pow2<32>(part);
      const int pv = rl >> 1;
      if ((rl & 1) == 0) red[buf][wave][pv < 16 ? 16 * h + pv : R + 16 * h + (pv - 16)] = tot;
    }
    lds_barrier();
    const int li = rl & (R - 1);  // row li on lanes li, li + R, ...
    // The sum of squares is over every wave (the whole d), the dot product
    // over the waves of this wave's head (H heads of W / H whole waves).
    float ss = 0.f, dt = 0.f;
    for (int w2 = 0; w2 < W; ++w2) ss += red[buf][w2][li];
    for (int w2 = hw0; w2 < hw0 + wph; ++w2) dt += red[buf][w2][R + li];
    // 3. scores and the online depth softmax
    const bool valid = tl * R + li < n_src;
    const float s = valid ? dt / sqrtf(ss * inv_d + a.eps) : -INFINITY;
    const float m_new = fmaxf(m, group_max<R>(s));
    const float scale = expf(m - m_new);  // 0 for the first tile (m = -inf)
    const float e = valid ? expf(s - m_new) : 0.f;
    lsum = lsum * scale + group_sum<R>(e);
    m = m_new;
#pragma unroll
    for (int c = 0; c < C; ++c) acc[c] *= scale;
    // 4. the weighted sum, refilling each row after its last use
#pragma unroll
    for (int k = 0; k < R; ++k) {
      // Unpack the row again: the fp32 copy from step 1 would need 256
      // registers across the barrier.
      float x[C];
      piece_unpack(piece_opaque(v[k]), x);
      // Past the last token, and for rows past n_src, the load reads nothing.
      v[k] = piece_ld<C>(row(pl, ns, tr, rn0 + k), coff, more && rn0 + k < ns ? 0x7fffffff : 0);
      const float al = read_lane(e, k);
#pragma unroll
      for (int c = 0; c < C; ++c) acc[c] = fmaf(al, x[c], acc[c]);
      __builtin_amdgcn_sched_barrier(0);  // one row's floats at a time
    }
    buf ^= 1;
    if (last) {
      const float inv = 1.0f / lsum;
      float o[C];
#pragma unroll
      for (int c = 0; c < C; ++c) o[c] = acc[c] * inv;
      piece_st(out + t * d, coff, 0x7fffffff, o);
      m = -INFINITY;
      lsum = 0.f;
#pragma unroll
      for (int c = 0; c < C; ++c) acc[c] = 0.f;
      tl = 0;
      t = tn;
    } else {
      ++tl;
    }
  }
}

// The kernel a call runs, as (tiles, channels per thread, rows per tile):
// tiles of 8 channels (16 rows for up to 16 sources, else 32) need heads of
// whole 512-channel waves and d <= 4096; 64-row tiles of 4 channels take up to
// 64 sources in one tile, heads of whole 256-channel waves and d <= 2048.
// {0, 0, 0}: none.
struct OnePick {
  int nt, c, r;
};
OnePick one_pick(const FullArgs& a) {
  if (!(a.H == 1 || a.H == 2 || a.H == 4 || a.H == 8) || a.d < 512 || a.d % 512 != 0) return {0, 0, 0};
  if (a.n_src < 1 || a.n_src > 64) return {0, 0, 0};
  const bool c8 = (a.d / a.H) % 512 == 0 && a.d <= 8 * 64 * kOMaxW;
  const bool c4 = (a.d / a.H) % 256 == 0 && a.d <= 4 * 64 * kOMaxW;
  if (a.n_src <= 16 && c8) return {1, 8, 16};
  if (a.n_src <= 32) return c8 ? OnePick{1, 8, 32} : (c4 ? OnePick{1, 4, 64} : OnePick{0, 0, 0});
  if (c4 && (kOneRows64 || !c8)) return {1, 4, 64};
  return c8 ? OnePick{2, 8, 32} : OnePick{0, 0, 0};
}

}  // namespace

bool full_one_ok(const FullArgs& a) {
  auto al16 = [](const void* p) { return p == nullptr || ((uintptr_t)p & 15u) == 0; };
  return a.dtype == kBF16 && a.n_dst == 1 && a.T >= 1 && one_pick(a).nt != 0 && al16(a.src) && al16(a.out) &&
         al16(a.w) && al16(a.gain);
}

namespace {
template <int NT, int C, int R>
hipError_t launch_one(const FullArgs& a, hipStream_t st) {
  const int B = (int)(a.d / C);
  int per_cu = 0;
  const hipError_t e = blocks_per_cu(reinterpret_cast<const void*>(k_full_one<NT, C, R>), B, &per_cu);
  if (e != hipSuccess) return e;
  int64_t grid = (int64_t)num_cus() * (per_cu < 1 ? 1 : per_cu);
  if (grid > a.T) grid = a.T;
  hipLaunchKernelGGL((k_full_one<NT, C, R>), dim3((unsigned)grid), dim3((unsigned)B), 0, st, a);
  return hipGetLastError();
}
}  // namespace

hipError_t launch_full_one(const FullArgs& a, hipStream_t st) {
  const OnePick p = one_pick(a);
  if (p.c == 4) return launch_one<1, 4, 64>(a, st);
  if (p.r == 16) return launch_one<1, 8, 16>(a, st);
  return p.nt == 2 ? launch_one<2, 8, 32>(a, st) : launch_one<1, 8, 32>(a, st);
}

}  // namespace attnres
