// Full AttnRes backward for one destination over up to 32 sources (gfx950,
// bf16 I/O, one head): the backward of the call a model makes per sublayer
// (b-lab.team summary §1 for the forward; the gradient is the chain rule
// through it).  Per token, with p_i = q . v_i, r_i = 1 / sqrt(mean(v_i^2) +
// eps), s_i = r_i p_i, alpha = softmax(s) and a_i = dout . v_i:
//   ds_i  = alpha_i (a_i - sum_m alpha_m a_m)
//   dv_i  = alpha_i dout + ds_i r_i q - ds_i p_i r_i^3 / d * v_i
//   Z    += sum_i ds_i r_i v_i            (dw = g * Z, dgain = w * Z)
// Three dot products per source row over d, then elementwise work: far too
// little arithmetic for the matrix cores, so this runs on the vector units
// and reads each source row and the token's dout row once.
//
// One workgroup of d / 8 threads owns one token at a time; thread tid owns
// channels 8 tid .. 8 tid + 7.  The token's 32 source rows sit in registers
// (16-byte buffer loads, one register quad per row; a row past n_src has a
// zero-record descriptor, so it is never read and its gradient never
// written):
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
#include "xlane.hpp"

namespace attnres {
namespace {

constexpr int kBTile = 32;    // source rows held in registers
constexpr int kBMaxW = 8;     // waves per workgroup at most (d <= 4096)
constexpr int kBSlabs = 1024; // workgroups (and Z slabs) at most
constexpr int kBRing = 8;     // accumulate: old d_src rows in flight ahead of their use
constexpr int kAll = 0x7fffffff;

template <bool ACC>
__global__ __launch_bounds__(512, 2) void k_full_bwd_one(FullBwdArgs a, float* zs) {
  __shared__ float red[2][kBMaxW][3 * kBTile];  // per buffer and wave: sums of squares, q . v, dout . v
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int W = (int)blockDim.x >> 6;
  const int d = (int)a.d, n_src = (int)a.n_src;
  const int64_t T = a.T, plane = T * d;
  const bf16_t* src = static_cast<const bf16_t*>(a.src);
  const bf16_t* dout = static_cast<const bf16_t*>(a.dout);
  bf16_t* dsrc = static_cast<bf16_t*>(a.d_src);
  const uint32_t coff = (uint32_t)tid * 16u;  // this thread's byte offset in a row
  // 1/d is read from LDS where it is used: a register copy held across the
  // token loop gets spilled.  (Written before the loop; every read follows
  // the loop's barrier.)
  __shared__ float lds_inv_d;
  if (tid == 0) lds_inv_d = 1.0f / (float)d;

  float q[8];  // q = w * g of the destination, for this thread's channels
  if (a.gain != nullptr)
    fold_q8<true>(a.w + 8 * tid, a.gain + 8 * tid, q);
  else
    fold_q8<false>(a.w + 8 * tid, nullptr, q);
  float z[8];
#pragma unroll
  for (int c = 0; c < 8; ++c) z[c] = 0.f;

  // Element offset of row r of token t (a row past n_src takes the last real
  // row's address, which its zero-record access never touches), from opaque
  // scalar copies of the plane size and the source count taken per token.
  auto row = [&](int64_t pl, int ns, int64_t t, int r) { return (int64_t)(r < ns ? r : ns - 1) * pl + t * d; };
  uint4 v[kBTile], go;
  int64_t t = blockIdx.x;
  if (t < T) {
#pragma unroll
    for (int k = 0; k < kBTile; ++k) v[k] = ld16_rec(src + row(plane, n_src, t, k), coff, k < n_src ? kAll : 0);
    go = ld16_rec(dout + t * d, coff);
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
    for (int h = 0; h < 2; ++h) {
      float part[kBTile];
#pragma unroll
      for (int k = 0; k < 16; ++k) {
        float x[8];
        unpack_bf8(v[16 * h + k], x);
        float ss = 0.f, p = 0.f;
#pragma unroll
        for (int c = 0; c < 8; ++c) {
          ss = fmaf(x[c], x[c], ss);
          p = fmaf(q[c], x[c], p);
        }
        part[k] = ss;
        part[16 + k] = p;
      }
      const float tot = transpose_reduce_pow2<kBTile>(part);
      if ((rl & 1) == 0) red[buf][wave][pv < 16 ? 16 * h + pv : kBTile + 16 * h + (pv - 16)] = tot;
    }
    // ... and dout . v for the 32 rows
    {
      float g[8], part[kBTile];
      unpack_bf8(go, g);
#pragma unroll
      for (int k = 0; k < kBTile; ++k) {
        // Unpack the row afresh: sharing the unpacked rows with the loop above
        // would keep 256 floats live between the two.
        uint4 u = v[k];
        asm volatile("" : "+v"(u.x), "+v"(u.y), "+v"(u.z), "+v"(u.w));
        float x[8];
        unpack_bf8(u, x);
        float da = 0.f;
#pragma unroll
        for (int c = 0; c < 8; ++c) da = fmaf(g[c], x[c], da);
        part[k] = da;
      }
      const float tot = transpose_reduce_pow2<kBTile>(part);
      if ((rl & 1) == 0) red[buf][wave][2 * kBTile + pv] = tot;
    }
    // With accumulate, the first old d_src rows are read while the waves meet.
    uint4 ring[ACC ? kBRing : 1];
    if constexpr (ACC) {
#pragma unroll
      for (int k = 0; k < kBRing; ++k) ring[k] = ld16_rec(dsrc + row(pl, ns, t, k), coff, k < ns ? kAll : 0);
    }
    lds_barrier();

    // 2. the softmax and the coefficients, row li on lanes li and li + 32
    const int li = rl & (kBTile - 1);
    float ss = 0.f, p = 0.f, da = 0.f;
    for (int w2 = 0; w2 < W; ++w2) {
      ss += red[buf][w2][li];
      p += red[buf][w2][kBTile + li];
      da += red[buf][w2][2 * kBTile + li];
    }
    const bool valid = li < n_src;
    const float inv_d = lds_inv_d;
    const float r = 1.0f / sqrtf(ss * inv_d + a.eps);
    const float s = valid ? r * p : -INFINITY;
    const float mx = group_max<kBTile>(s);
    const float e = valid ? expf(s - mx) : 0.f;
    const float al = e / group_sum<kBTile>(e);
    const float ds = al * (da - group_sum<kBTile>(al * da));
    const float cq = ds * r;                       // coefficient of q in dv, and of v in Z
    const float cv = -ds * p * r * r * r * inv_d;  // coefficient of v in dv (through the RMS)

    // 3. d_src, row by row; each row's register then takes the next token's row
    float g[8];
    unpack_bf8(go, g);
#pragma unroll
    for (int k = 0; k < kBTile; ++k) {
      uint4 u = v[k];
      asm volatile("" : "+v"(u.x), "+v"(u.y), "+v"(u.z), "+v"(u.w));
      float x[8];
      unpack_bf8(u, x);
      v[k] = ld16_rec(src + row(pl, ns, tr, k), coff, more && k < ns ? kAll : 0);
      const float A = read_lane(al, k), B = read_lane(cq, k), C = read_lane(cv, k);
      float o[8];
#pragma unroll
      for (int c = 0; c < 8; ++c) {
        o[c] = fmaf(A, g[c], fmaf(B, q[c], C * x[c]));
        z[c] = fmaf(B, x[c], z[c]);
      }
      if constexpr (ACC) {
        float old[8];
        unpack_bf8(ring[k % kBRing], old);
#pragma unroll
        for (int c = 0; c < 8; ++c) o[c] += old[c];
        if (k + kBRing < kBTile)
          ring[k % kBRing] = ld16_rec(dsrc + row(pl, ns, t, k + kBRing), coff, k + kBRing < ns ? kAll : 0);
      }
      st16_rec(dsrc + row(pl, ns, t, k), coff, k < ns ? kAll : 0,
               make_uint4(pack_bf2(o[0], o[1]), pack_bf2(o[2], o[3]), pack_bf2(o[4], o[5]), pack_bf2(o[6], o[7])));
      __builtin_amdgcn_sched_barrier(0);  // one row's floats at a time
    }
    // The next token's dout row, first needed after its rows' first pass.
    go = ld16_rec(dout + tr * d, coff, more ? kAll : 0);
    buf ^= 1;
    t = tn;
  }
  // This workgroup's slab of Z (zeros if it had no token): 32 bytes per
  // thread, at twice the thread's bf16 row offset.
  float* zrow = zs + (int64_t)blockIdx.x * d;
  uint32_t zoff = coff;
  asm volatile("" : "+v"(zoff));  // formed here, not held across the loop
  zoff *= 2;
  st16_rec(zrow, zoff, kAll, make_uint4(__float_as_uint(z[0]), __float_as_uint(z[1]), __float_as_uint(z[2]), __float_as_uint(z[3])));
  st16_rec(zrow, zoff + 16, kAll, make_uint4(__float_as_uint(z[4]), __float_as_uint(z[5]), __float_as_uint(z[6]), __float_as_uint(z[7])));
}

bool one_shape(int64_t n_src, int64_t n_dst, int64_t d, int H) {
  return H == 1 && n_dst == 1 && n_src >= 1 && n_src <= kBTile && d >= 512 && d % 512 == 0 && d <= 8 * 64 * kBMaxW;
}

int64_t one_slabs(int64_t T) { return T < kBSlabs ? T : kBSlabs; }

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
  const int B = (int)(a.d / 8);
  auto kern = a.accumulate ? k_full_bwd_one<true> : k_full_bwd_one<false>;
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

}  // namespace attnres
