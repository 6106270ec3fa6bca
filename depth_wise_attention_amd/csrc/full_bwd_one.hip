// Full AttnRes backward for one destination over up to 64 sources (gfx950,
// bf16 I/O): the backward of the call a model makes per sublayer (b-lab.team
// summary §1 for the forward; the gradient is the chain rule through it).
// Per token, with p_i = q . v_i, r_i = 1 / sqrt(mean(v_i^2) + eps),
// s_i = r_i p_i, alpha = softmax(s) and a_i = dout . v_i:
//   ds_i  = alpha_i (a_i - sum_m alpha_m a_m)
//   dv_i  = alpha_i dout + ds_i r_i q - ds_i p_i r_i^3 / d * v_i
//   Z    += sum_i ds_i r_i v_i            (dw = g * Z, dgain = w * Z)
// With H heads (chatpaper MHAR abstract) p, a, alpha and ds are per head over
// the head's channels, r is over the whole d, and the v term of dv sums
// ds p over the heads.
// Three dot products per source row over d, then elementwise work: far too
// little arithmetic for the matrix cores, so this runs on the vector units
// and reads each source row and the token's dout row once.
//
// One workgroup of d / C threads owns one token at a time; thread tid owns
// channels C tid .. C tid + C - 1.  All R source rows of the token sit in
// registers: R = 16 or 32 rows of 8 channels (four registers a row) for up to
// 16 or 32 sources, or 64 rows of 4 channels (two a row) for 33 .. 64.  A row
// past n_src
// has a zero-record descriptor, so it is never read and its gradient never
// written:
//   1. per row, the sum of squares, q . v and dout . v over the thread's
//      channels, reduced over the wave by transposing reductions and over the
//      waves through double-buffered LDS (one barrier per token);
//   2. the softmax and the three per-row coefficients, one row per lane;
//   3. per row, dv from the registers, stored as bf16; as each row is used
//      its register takes the next token's row.
// Z stays in registers across the workgroup's tokens and is written once as
// the workgroup's slab; a fixed-order sum over the slabs gives dw and dgain.
// With accumulate, the old d_src rows are read eight rows ahead of their use.
#include <math.h>

#include "common.hpp"
#include "launch.hpp"
#include "row_piece.hpp"
#include "xlane.hpp"

namespace attnres {
namespace {

constexpr int kBMaxW = 8;     // waves per workgroup at most
constexpr int kBSlabs = 1024; // workgroups (and Z slabs) at most
constexpr int kBRing = 8;     // accumulate: old d_src rows in flight ahead of their use
constexpr int kAll = 0x7fffffff;

template <bool ACC, int R, bool MH>
__global__ __launch_bounds__(512, 2) void k_full_bwd_one(FullBwdArgs a, float* zs) {
  constexpr int C = R == 64 ? 4 : 8;  // channels per thread
  typedef typename PieceOf<C>::type P;
  __shared__ float red[2][kBMaxW][3 * R];  // per buffer and wave: sums of squares, q . v, dout . v
  __shared__ float dsp[MH ? 2 : 1][MH ? kBMaxW : 1][R];  // heads: ds p per head and row
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int W = (int)blockDim.x >> 6;
  // Heads are runs of W / H whole waves: this wave's head and its first wave.
  const int wph = MH ? W / a.H : W, head = wave / wph, hw0 = head * wph;
  const int d = (int)a.d, n_src = (int)a.n_src;
  const int64_t T = a.T, plane = T * d;
  const bf16_t* src = static_cast<const bf16_t*>(a.src);
  const bf16_t* dout = static_cast<const bf16_t*>(a.dout);
  bf16_t* dsrc = static_cast<bf16_t*>(a.d_src);
  const uint32_t coff = (uint32_t)tid * (2u * C);  // this thread's byte offset in a row
  // 1/d is read from LDS where it is used: a register copy held across the
  // token loop gets spilled.  (Written before the loop; every read follows
  // the loop's barrier.)
  __shared__ float lds_inv_d;
  if (tid == 0) lds_inv_d = 1.0f / (float)d;

  float q[C];  // q = w * g of the destination, for this thread's channels
  if (a.gain != nullptr)
    fold_q<C>(a.w + C * tid, a.gain + C * tid, q);
  else
    fold_q<C>(a.w + C * tid, nullptr, q);
  float z[C];
#pragma unroll
  for (int c = 0; c < C; ++c) z[c] = 0.f;

  // Element offset of row r of token t (a row past n_src takes the last real
  // row's address, which its zero-record access never touches), from opaque
  // scalar copies of the plane size and the source count taken per token.
  auto row = [&](int64_t pl, int ns, int64_t t, int r) { return (int64_t)(r < ns ? r : ns - 1) * pl + t * d; };
  P v[R], go;
  int64_t t = blockIdx.x;
  if (t < T) {
#pragma unroll
    for (int k = 0; k < R; ++k) v[k] = piece_ld<C>(src + row(plane, n_src, t, k), coff, k < n_src ? kAll : 0);
    go = piece_ld<C>(dout + t * d, coff, kAll);
  }
  int buf = 0;
#pragma unroll 1
  while (t < T) {
    const int64_t tn = t + gridDim.x;
    const bool more = tn < T;
    const int64_t tr = more ? tn : t;  // a real token for the refill addresses
    int64_t pl = plane;
    int ns = n_src;
    asm volatile("" : "+s"(pl), "+s"(ns));
    // The lane id from mbcnt, which reads no register: rematerialised per
    // token instead of held (and spilled) across the loop.
    const int rl = (int)__builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
    const int pv = rl >> 1;  // after a 32-value transposing reduction lane L holds value L >> 1

    // 1. sums of squares and q . v, 16 rows at a time (32 partials)
#pragma unroll
    for (int h = 0; h < R / 16; ++h) {
      float part[32];
#pragma unroll
      for (int k = 0; k < 16; ++k) {
        float x[C];
        piece_unpack(v[16 * h + k], x);
        float ss = 0.f, p = 0.f;
#pragma unroll
        for (int c = 0; c < C; ++c) {
          ss = fmaf(x[c], x[c], ss);
          p = fmaf(q[c], x[c], p);
        }
        part[k] = ss;
        part[16 + k] = p;
      }
      const float tot = transpose_reduce_pow2<32>(part);
      if ((rl & 1) == 0) red[buf][wave][pv < 16 ? 16 * h + pv : R + 16 * h + (pv - 16)] = tot;
    }
    // ... and dout . v, 32 rows at a time (a 16-row tile pads with zeros)
    {
      float g[C];
      piece_unpack(go, g);
#pragma unroll
      for (int h = 0; h < (R + 31) / 32; ++h) {
        float part[32];
#pragma unroll
        for (int k = 0; k < 32; ++k) {
          if (32 * h + k >= R) {
            part[k] = 0.f;
            continue;
          }
          // Unpack afresh: sharing the unpacked rows with the pass above
          // would keep 256 floats live between the two.
          float x[C];
          piece_unpack(piece_opaque(v[32 * h + k]), x);
          float da = 0.f;
#pragma unroll
          for (int c = 0; c < C; ++c) da = fmaf(g[c], x[c], da);
          part[k] = da;
        }
        const float tot = transpose_reduce_pow2<32>(part);
        if ((rl & 1) == 0 && 32 * h + pv < R) red[buf][wave][2 * R + 32 * h + pv] = tot;
      }
    }
    // With accumulate, the first old d_src rows are read while the waves meet.
    P ring[ACC ? kBRing : 1];
    if constexpr (ACC) {
#pragma unroll
      for (int k = 0; k < kBRing; ++k) ring[k] = piece_ld<C>(dsrc + row(pl, ns, t, k), coff, k < ns ? kAll : 0);
    }
    lds_barrier();

    // 2. the softmax and the coefficients, row li on lane li (and li + 32 when R = 32)
    const int li = rl & (R - 1);
    // The sum of squares is over every wave (the whole d); the products with
    // q and dout are over this head's waves.
    float ss = 0.f, p = 0.f, da = 0.f;
    for (int w2 = 0; w2 < W; ++w2) ss += red[buf][w2][li];
    for (int w2 = hw0; w2 < hw0 + wph; ++w2) {
      p += red[buf][w2][R + li];
      da += red[buf][w2][2 * R + li];
    }
    const bool valid = li < n_src;
    const float inv_d = lds_inv_d;
    const float r = 1.0f / sqrtf(ss * inv_d + a.eps);
    const float s = valid ? r * p : -INFINITY;
    const float mx = group_max<R>(s);
    const float e = valid ? expf(s - mx) : 0.f;
    const float al = e / group_sum<R>(e);
    const float ds = al * (da - group_sum<R>(al * da));
    const float cq = ds * r;  // coefficient of q in dv, and of v in Z
    // The coefficient of v in dv comes through the RMS, which every head
    // shares: -r^3 / d times the sum over heads of ds p, exchanged through LDS
    // (a second barrier) when there are several.
    float dsp_all = ds * p;
    if constexpr (MH) {
      if (wave == hw0 && rl < R) dsp[buf][head][li] = dsp_all;
      lds_barrier();
      dsp_all = 0.f;
      for (int h2 = 0; h2 < a.H; ++h2) dsp_all += dsp[buf][h2][li];
    }
    const float cv = -dsp_all * r * r * r * inv_d;

    // 3. d_src, row by row; each row's register then takes the next token's row
    float g[C];
    piece_unpack(go, g);
#pragma unroll
    for (int k = 0; k < R; ++k) {
      float x[C];
      piece_unpack(piece_opaque(v[k]), x);
      v[k] = piece_ld<C>(src + row(pl, ns, tr, k), coff, more && k < ns ? kAll : 0);
      const float A = read_lane(al, k), B = read_lane(cq, k), Cv = read_lane(cv, k);
      float o[C];
#pragma unroll
      for (int c = 0; c < C; ++c) {
        o[c] = fmaf(A, g[c], fmaf(B, q[c], Cv * x[c]));
        z[c] = fmaf(B, x[c], z[c]);
      }
      if constexpr (ACC) {
        float old[C];
        piece_unpack(ring[k % kBRing], old);
#pragma unroll
        for (int c = 0; c < C; ++c) o[c] += old[c];
        if (k + kBRing < R)
          ring[k % kBRing] = piece_ld<C>(dsrc + row(pl, ns, t, k + kBRing), coff, k + kBRing < ns ? kAll : 0);
      }
      piece_st(dsrc + row(pl, ns, t, k), coff, k < ns ? kAll : 0, o);
    }
    // The next token's dout row, first needed after its rows' first pass.
    go = piece_ld<C>(dout + tr * d, coff, more ? kAll : 0);
    buf ^= 1;
    t = tn;
  }
  // This workgroup's slab of Z (zeros if it had no token): 4 C bytes per
  // thread, at twice the thread's bf16 row offset.
  float* zrow = zs + (int64_t)blockIdx.x * d;
  uint32_t zoff = coff;
  asm volatile("" : "+v"(zoff));  // formed here, not held across the loop
  zoff *= 2;
#pragma unroll
  for (int k = 0; k < C; k += 4)
    st16_rec(zrow, zoff + 4 * k, kAll,
             make_uint4(__float_as_uint(z[k]), __float_as_uint(z[k + 1]), __float_as_uint(z[k + 2]),
                        __float_as_uint(z[k + 3])));
}

// Rows held per thread: 16 (8 channels, half the registers, so more tokens
// in flight per CU) for up to 16 sources, 32 (8 channels) for up to 32, both
// with d up to 4096; 64 (4 channels, d up to 2048) for 33 .. 64.
int one_rows(int64_t n_src) { return n_src > 32 ? 64 : (n_src > 16 ? 32 : 16); }

bool one_shape(int64_t n_src, int64_t n_dst, int64_t d, int H) {
  if (n_dst != 1 || n_src < 1 || n_src > 64 || d < 512 || d % 512 != 0) return false;
  const int64_t wave_ch = (one_rows(n_src) == 64 ? 4 : 8) * 64;  // channels per wave
  if (d > wave_ch * kBMaxW) return false;
  // Heads of whole waves.
  return H == 1 || ((H == 2 || H == 4 || H == 8) && (d / H) % wave_ch == 0);
}

int64_t one_slabs(int64_t T) { return T < kBSlabs ? T : kBSlabs; }

template <int R>
hipError_t launch_rows(const FullBwdArgs& a, const float** slabs, int64_t* n_slabs, hipStream_t st) {
  const int B = (int)(a.d / (R == 64 ? 4 : 8));
  auto kern = a.H > 1 ? (a.accumulate ? k_full_bwd_one<true, R, true> : k_full_bwd_one<false, R, true>)
                      : (a.accumulate ? k_full_bwd_one<true, R, false> : k_full_bwd_one<false, R, false>);
  int per_cu = 0;
  const hipError_t e = blocks_per_cu(reinterpret_cast<const void*>(kern), B, &per_cu);
  if (e != hipSuccess) return e;
  int64_t grid = (int64_t)num_cus() * (per_cu < 1 ? 1 : per_cu);
  if (grid > one_slabs(a.T)) grid = one_slabs(a.T);
  hipLaunchKernelGGL(kern, dim3((unsigned)grid), dim3((unsigned)B), 0, st, a, a.zslots);
  *slabs = a.zslots;
  *n_slabs = grid;
  return hipGetLastError();
}

}  // namespace

size_t full_bwd_one_workspace_bytes(int64_t n_src, int64_t n_dst, int64_t T, int64_t d, int H) {
  return one_shape(n_src, n_dst, d, H) ? (size_t)one_slabs(T) * (size_t)d * 4 : 0;
}

bool full_bwd_one_ok(const FullBwdArgs& a) {
  auto al16 = [](const void* p) { return p == nullptr || ((uintptr_t)p & 15u) == 0; };
  if (a.dtype != kBF16 || a.T < 1 || !one_shape(a.n_src, a.n_dst, a.d, a.H)) return false;
  if (a.zslots == nullptr || a.ws_bytes < full_bwd_one_workspace_bytes(a.n_src, a.n_dst, a.T, a.d, a.H)) return false;
  return al16(a.src) && al16(a.dout) && al16(a.d_src) && al16(a.zslots) && al16(a.w) && al16(a.gain);
}

hipError_t launch_full_bwd_one(const FullBwdArgs& a, const float** slabs, int64_t* n_slabs, hipStream_t st) {
  switch (one_rows(a.n_src)) {
    case 16: return launch_rows<16>(a, slabs, n_slabs, st);
    case 32: return launch_rows<32>(a, slabs, n_slabs, st);
    default: return launch_rows<64>(a, slabs, n_slabs, st);
  }
}

}  // namespace attnres
